// Host-side helpers shared by the C entry points: thread-local error text and
// argument validation.  No device code.
#pragma once

#include <stdarg.h>
#include <stdint.h>

#include "lazy_attn.h"

namespace lazy {

// Records a formatted message for lazy_last_error() and returns `st`.
lazy_status fail(lazy_status st, const char* fmt, ...);
void clear_error();

// Geometry checks shared by every device call.
lazy_status check_geom(const lazy_geom* g);
// Positional-descriptor checks (needs_rotation: the call reads cos/sin).
lazy_status check_pos(const lazy_geom* g, const lazy_pos_desc* p);

}  // namespace lazy
