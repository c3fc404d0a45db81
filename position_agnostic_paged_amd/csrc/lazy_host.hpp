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

// The document pass of the document-major decode (rows = reads of one shared
// document x the query group).  bf16 runs the LDS-staged pass: a workgroup of
// kDocPassLdsWaves waves, kDocPassLdsRb blocks of 16 rows each, copies each
// tile pair once for all its rows.  fp32 runs the per-wave pass,
// LAZY_DOCPASS_RB128 (dh 128) or 4 (dh 64) row blocks per wave.
#ifndef LAZY_DOCPASS_RB128
#define LAZY_DOCPASS_RB128 2
#endif
#ifndef LAZY_DOCPASS_LDS_WAVES
#define LAZY_DOCPASS_LDS_WAVES 4
#endif
#ifndef LAZY_DOCPASS_LDS_RB
#define LAZY_DOCPASS_LDS_RB 2
#endif
constexpr int kDocPassLdsWaves = LAZY_DOCPASS_LDS_WAVES;
constexpr int kDocPassLdsRb = LAZY_DOCPASS_LDS_RB;
#ifndef LAZY_DOCPASS_LDS
#define LAZY_DOCPASS_LDS 1  // 0: bf16 runs the per-wave pass too
#endif
inline bool docpass_uses_lds(const lazy_geom* g) { return LAZY_DOCPASS_LDS && g->dtype == LAZY_BF16; }
// 16-row blocks of one work item (a workgroup of the LDS pass, a wave of the
// per-wave pass); the planner and the launch agree through this one function.
inline int docpass_row_blocks(const lazy_geom* g) {
  if (docpass_uses_lds(g)) return kDocPassLdsWaves * kDocPassLdsRb;
  return g->head_dim == 128 ? LAZY_DOCPASS_RB128 : 4;
}

}  // namespace lazy
