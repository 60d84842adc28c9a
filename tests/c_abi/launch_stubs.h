// Records of the host-only launcher stand-ins (launch_stubs.cpp).
#pragma once

#include "csa_internal.h"

namespace csa {

struct StubLog {
  IndexParams index{};
  TopkParams topk{};
  AttnParams attn{};
  int n_index = 0, n_topk = 0, n_index_topk = 0, n_index_topk_prefill = 0, n_attn = 0;
};
extern StubLog g_stub;

}  // namespace csa
