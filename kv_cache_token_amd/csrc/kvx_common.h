// Internal helpers shared by the library's translation units (not part of the ABI).
#pragma once

#include <stdint.h>

#include "kvevict.h"

namespace kvx {

// Records a message for kvx_last_error() and returns `code`.
int set_error(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the message (called on entry of every ABI function).
void clear_error();

}  // namespace kvx
