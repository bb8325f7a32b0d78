// Parameter blocks recorded by the launch stubs of the AddressSanitizer host
// build (launch_stubs.cpp).
#pragma once

#include "beam_kernels.h"
#include "kv_layout.h"

namespace stub {
struct Record {
  int calls = 0;
  int grid_a = 0, grid_b = 0;
  beam::PrologueParams prologue{};
  beam::AppendParams append{};
  beam::DecodeQParams decode_q{};
  beam::PrefillParams prefill{};
  beam::DecodeParams decode{};
  beam::CombineParams combine{};
};
extern Record last;
}  // namespace stub
