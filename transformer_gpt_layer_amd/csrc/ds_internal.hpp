// ds_internal.hpp -- host-side objects shared by the C ABI translation units.
#pragma once
#include <string>

#include "../../include/ds_layer.h"

struct ds_layer {
  ds_layer_desc desc;
  ds_layer_weights w;
};

namespace ds {
// Sets the calling thread's last-error message and returns `code`.
int set_error(int code, const char* fmt, ...);
}  // namespace ds
