// ds_internal.hpp -- host-side objects shared by the C ABI translation units.
#pragma once
#include <string>

#include "../../include/ds_layer.h"

struct ds_layer {
  ds_layer_desc desc;
  ds_layer_weights w;
  // MFMA tile configuration forced for every GEMM of this layer (-1: chosen per product). Read from
  // the DS_GEMM_CONFIG environment variable at create time; for tests that must run each
  // configuration on shapes where the automatic choice would not take it.
  int gemm_cfg = -1;
};

namespace ds {
// Sets the calling thread's last-error message and returns `code`.
int set_error(int code, const char* fmt, ...);
}  // namespace ds
