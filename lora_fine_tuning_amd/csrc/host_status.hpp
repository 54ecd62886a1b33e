// Host-side status reporting shared by the C-ABI translation units: sets the
// thread-local message read by lora_last_error_message() and returns `st`.
#pragma once

#include "lora_fused.h"

namespace lora {
lora_status host_fail(lora_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
}  // namespace lora
