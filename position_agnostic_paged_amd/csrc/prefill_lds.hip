// LDS-staged prefill over a position-agnostic paged cache (bf16, gfx950).
//
// Same computation as the per-wave prefill (LazyAttention notes,
// papernotes.org, "Key designs": compute-bound prefill with the document
// offset applied inside the fused kernel), organised for CDNA4:
//
//   * a workgroup = NW waves x RB blocks of 16 GQA-packed query rows of one
//     (request, KV head); all waves consume the same tile pairs;
//   * each tile pair (K 2 x 16 x dh, V 2 x dh x 16, plus the two cos/sin
//     rows of the pair's document offsets) is copied once per workgroup
//     from HBM into LDS with direct global->LDS loads (no registers), into a
//     ring of kStages buffers, so kStages-1 pairs are in flight while one is
//     consumed by the MFMAs;
//   * LDS rows are XOR-swizzled at 16-byte granularity so the per-lane
//     fragment reads (16 B of a K row, 8 B of a V channel row) are free of
//     bank conflicts;
//   * the query is re-rotated by -Delta once per document from the raw
//     query parked in LDS and the cos/sin row in the stage, so the loop
//     issues no global load besides the stage copies (keeping the counted
//     waits on the copies exact);
//   * the softmax is trimmed for the matrix cores: pairs of two full
//     document tiles (the bulk of a long context) skip masking; the row max
//     is taken on raw scores against a per-row threshold, so the cross-lane
//     reduction and the rescale only run when some row's maximum grows by
//     more than 2^LAZY_RESCALE_SLACK; the scale folds into the exponent's
//     FMA; row sums come from one extra MFMA against a ones operand (the
//     sum of exactly the bf16 weights that multiply V).
#include "attn_common.hpp"

#ifndef LAZY_PREFILL_LDS_WAVES
#define LAZY_PREFILL_LDS_WAVES 8  // waves per workgroup (8: two per SIMD, 4: one)
#endif

namespace lazy {

constexpr int kStages = 4;  // LDS ring of tile pairs

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

template <int DH, bool ROT, int NW>
struct StageGeom {
  static constexpr int kTile = kBlock * DH * 2;      // bytes of one 16 x dh bf16 tile
  static constexpr int kChunksPerRow = DH / 8;       // 16-byte chunks in a K row
  static constexpr int kK = 0;                       // two K tiles
  static constexpr int kV = 2 * kTile;               // two V tiles
  static constexpr int kCS = 4 * kTile;              // two cos/sin rows (fp32 [dh])
  static constexpr int kBytes = 4 * kTile + (ROT ? 2 * DH * 4 : 0);
  static constexpr int kKChunks = 2 * kTile / 16;    // 16-B chunks of the K pair (same for V)
  static constexpr int kCopies = 2 * kKChunks / (NW * 64);  // K + V copies per thread
  static constexpr int kLoads = kCopies + (ROT ? 1 : 0);    // copies per wave per stage
  // every wave issues the same number of copies (the counted waits rely on
  // it) and no wave's 64 chunks straddle the K / V boundary
  static_assert(kCopies >= 1 && (2 * kKChunks) % (NW * 64) == 0 && kKChunks % 64 == 0, "stage copy shape");
};

typedef const __attribute__((address_space(4))) uint64_t* const_words;

template <int DH, int KIND, bool DEFER, int RB, int NW>
struct LdsPrefill {
  using F8 = bf16x8;
  using F4 = bf16x4;
  static constexpr int NC = DH / 32;  // contraction chunks of QK^T
  static constexpr int NV = DH / 16;  // 16-channel blocks of the output
  static constexpr bool kRot = (KIND != kAlibi) && DEFER;
  using SG = StageGeom<DH, kRot, NW>;

  const AttnArgs& a;
  unsigned char* lds;
  int tid, lane, wave, r, g, kvh, sb, se, nctx;
  // The tile table is read-only for the kernel's lifetime, so it is read
  // through the constant address space: scalar loads, counted apart from the
  // stage copies.
  const_words words;

  // tile words of pair p, decoded with the device-side guards
  __device__ __forceinline__ void pair_meta(int p, TileMeta (&mt)[2], int (&delta)[2], bool (&priv)[2]) const {
    const int ia = sb + 2 * p;
    mt[0] = unpack_word(words[ia]);
    mt[1] = unpack_word(words[min(ia + 1, se - 1)]);
    if (ia + 1 >= se) mt[1].mask = 0u;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      priv[x] = ia + x >= nctx;
      if (mt[x].block >= a.num_blocks || mt[x].block < 0) {  // never dereference outside the pool
        mt[x].block = 0;
        mt[x].mask = 0u;
      }
      delta[x] = (kRot && !priv[x]) ? mt[x].offset : 0;
      if (kRot && delta[x] >= a.max_pos) {  // outside the table: drop the tile
        mt[x].mask = 0u;
        delta[x] = 0;
      }
    }
  }

  // copy pair p into stage buffer p % kStages (every wave issues SG::kLoads copies)
  __device__ __forceinline__ void issue(int p) const {
    TileMeta mt[2];
    int delta[2];
    bool priv[2];
    pair_meta(p, mt, delta, priv);
    unsigned char* st = lds + (p % kStages) * SG::kBytes;
    const bf16* kc = reinterpret_cast<const bf16*>(a.k_cache);
    const bf16* vc = reinterpret_cast<const bf16*>(a.v_cache);
#pragma unroll
    for (int i = 0; i < SG::kCopies; ++i) {
      // chunk ci of the stage's K pair, then V pair; the LDS slot of a copy
      // is the wave's base plus 16 B per lane, i.e. stage offset 16 * ci
      const int ci = i * NW * 64 + tid;
      const bool is_v = ci >= SG::kKChunks;  // wave-uniform
      const int cv = is_v ? ci - SG::kKChunks : ci;
      const int x = cv / (SG::kTile / 16);
      const int cc = cv % (SG::kTile / 16);
      const int blk = x ? mt[1].block : mt[0].block;
      const int64_t base = ((int64_t)blk * a.hkv + kvh) * (kBlock * DH);
      const bf16* src;
      if (!is_v) {
        const int row = cc / SG::kChunksPerRow, pos = cc % SG::kChunksPerRow;
        src = kc + base + row * DH + (pos ^ (row % SG::kChunksPerRow)) * 8;
      } else {  // V rows are channels of 16 tokens = 2 chunks
        const int row = cc >> 1, pos = cc & 1;
        src = vc + base + row * kBlock + (pos ^ ((row >> 3) & 1)) * 8;
      }
      __builtin_amdgcn_global_load_lds(src, st + (i * NW + wave) * 64 * 16, 16, 0, 0);
    }
    if (kRot) {
      // the two cos/sin rows: DH/4 chunks each; wave w copies its share (lane-masked)
      constexpr int kCsChunks = 2 * (DH / 4);
      constexpr int kPerWave = kCsChunks / NW;
      static_assert(kPerWave >= 1 && kCsChunks <= 64, "cos/sin copy shape");
      if (lane >= wave * kPerWave && lane < (wave + 1) * kPerWave) {
        const int x = lane / (DH / 4);
        const int j = lane % (DH / 4);
        const int d = x ? delta[1] : delta[0];
        const float* src = a.cos_sin + (int64_t)d * DH + j * 4;  // a table is required (host checks)
        __builtin_amdgcn_global_load_lds(src, st + SG::kCS, 16, 0, 0);
      }
    }
  }

  // the wave's parked raw query fragment (b, c)
  __device__ __forceinline__ F8 raw_at(const unsigned char* raw, int b, int c) const {
    return *reinterpret_cast<const F8*>(raw + ((b * NC + c) * 64 + lane) * 16);
  }

  // q' = R_{-delta} q from the parked raw query and the stage's cos/sin row x
  __device__ __forceinline__ void rotate(F8 (&qr)[RB][NC], const unsigned char* raw, const unsigned char* st, int x,
                                         int delta) const {
    if (delta == 0) {
#pragma unroll
      for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int c = 0; c < NC; ++c) qr[b][c] = raw_at(raw, b, c);
      return;
    }
    const float* row = reinterpret_cast<const float*>(st + SG::kCS) + x * DH;
    if (KIND == kHalf) {
#pragma unroll
      for (int c = 0; c < NC / 2; ++c) {
        const float* cp = row + 32 * c + 8 * g;
        const f32x4 c0 = *reinterpret_cast<const f32x4*>(cp), c1 = *reinterpret_cast<const f32x4*>(cp + 4);
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(cp + DH / 2);
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(cp + DH / 2 + 4);
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const F8 lo = raw_at(raw, b, c), hi = raw_at(raw, b, c + NC / 2);
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const float cs = t < 4 ? c0[t] : c1[t - 4], sn = t < 4 ? s0[t] : s1[t - 4];
            const float x1 = (float)lo[t], x2 = (float)hi[t];
            qr[b][c][t] = (bf16)(x1 * cs + x2 * sn);
            qr[b][c + NC / 2][t] = (bf16)(x2 * cs - x1 * sn);
          }
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const float* cp = row + 16 * c + 4 * g;
        const f32x4 c0 = *reinterpret_cast<const f32x4*>(cp), s0 = *reinterpret_cast<const f32x4*>(cp + DH / 2);
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const F8 xr = raw_at(raw, b, c);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float x1 = (float)xr[2 * u], x2 = (float)xr[2 * u + 1];
            qr[b][c][2 * u] = (bf16)(x1 * c0[u] + x2 * s0[u]);
            qr[b][c][2 * u + 1] = (bf16)(x2 * c0[u] - x1 * s0[u]);
          }
        }
      }
    }
  }
};

template <int DH, int KIND, bool DEFER, int RB, int NW>
__global__ __launch_bounds__(64 * NW, 1) void prefill_lds_kernel(AttnArgs a) {
  using P = LdsPrefill<DH, KIND, DEFER, RB, NW>;
  using F8 = typename P::F8;
  using F4 = typename P::F4;
  constexpr int NC = P::NC;
  constexpr int NV = P::NV;
  using SG = typename P::SG;
  extern __shared__ __align__(16) unsigned char lds_buf[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int req = blockIdx.z;
  const int kvh = blockIdx.y;
  const int row_tile = blockIdx.x / a.num_splits;
  const int split = blockIdx.x % a.num_splits;

  const int q0 = a.q_start[req];
  int nq = a.q_start[req + 1] - q0;
  nq = min(nq, a.max_q_len);
  nq = max(0, min(nq, a.rows_bound / a.hq - q0));
  const int nrows = nq * a.group;
  const int t0 = a.tile_start[req];
  const int nt = a.tile_start[req + 1] - t0;
  int sb, se;
  // workgroup-uniform exits only (barriers follow)
  if (row_tile * NW * RB * 16 >= nrows) return;
  if (!split_range(nt, a.chunk, a.num_splits, split, sb, se)) return;
  const int npairs = (se - sb + 1) >> 1;
  const int rb0 = (row_tile * NW + wave) * RB;
  const bool has_rows = rb0 * 16 < nrows;  // wave-uniform: waves without rows still copy tiles
  const int qpos0 = a.q_pos[req];

  P pl{a, lds_buf, tid, lane, wave, r, g, kvh, sb, se, a.ctx_tiles[req], (const_words)(a.tiles + t0)};

  // Query rows: row rho of the request is (token rho / G, head kvh*G + rho % G);
  // rows past the request's last are zero (computed, never stored).  The raw
  // query at its global position, the source of every re-rotation, is parked
  // in this wave's LDS area (fragment order, 16 B per lane).
  unsigned char* raw = lds_buf + kStages * SG::kBytes + wave * (RB * NC * 64 * 16);
  int qp[RB];
  float slope_raw[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int rho = (rb0 + b) * 16 + r;
    const bool ok = rho < nrows;
    const int qi = ok ? rho / a.group : 0;
    const int head = kvh * a.group + (ok ? rho % a.group : 0);
    qp[b] = qpos0 + qi;
    // ALiBi in the raw-score domain: bias / softmax scale
    slope_raw[b] = (KIND == kAlibi) ? a.slopes[head] * kLog2e / a.scale_log2 : 0.f;
    const bf16* qrow = reinterpret_cast<const bf16*>(a.q) + ((int64_t)(q0 + qi) * a.hq + head) * DH;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      F8 v = *reinterpret_cast<const F8*>(qrow + 32 * c + 8 * g);
      if (!ok) v = F8{};
      *reinterpret_cast<F8*>(raw + ((b * NC + c) * 64 + lane) * 16) = v;
    }
  }
  F8 qr[RB][NC];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int c = 0; c < NC; ++c) qr[b][c] = pl.raw_at(raw, b, c);
  int cur_delta = 0;

  f32x4 acc[RB][NV];
  f32x4 lsum[RB];  // row sums, replicated in the four registers
  float m_run[RB], negm[RB], thr[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
#pragma unroll
    for (int n = 0; n < NV; ++n) acc[b][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    lsum[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[b] = -INFINITY;  // log2-domain reference max
    negm[b] = 0.f;         // -m_run (0 while m_run is -inf)
    thr[b] = -INFINITY;    // raw score above which the reference must move
  }
  const float sl = a.scale_log2;
  F8 ones;
#pragma unroll
  for (int t = 0; t < 8; ++t) ones[t] = (bf16)1.f;

  // prologue: kStages - 1 pairs in flight
#pragma unroll
  for (int p = 0; p < kStages - 1; ++p)
    if (p < npairs) pl.issue(p);

  for (int p = 0; p < npairs; ++p) {
    // copies issued after pair p: min(kStages - 2, npairs - 1 - p) stages
    const int after = min(kStages - 2, npairs - 1 - p);
    if (after >= 2)
      wait_vmcnt<2 * SG::kLoads>();
    else if (after == 1)
      wait_vmcnt<SG::kLoads>();
    else
      wait_vmcnt<0>();
    // Every wave has waited for its own copies of pair p; the barrier makes
    // them complete for all waves and frees buffer (p - 1) % kStages.  A bare
    // s_barrier (compiler memory clobber only): a fenced __syncthreads would
    // also drain the copies of the later pairs still in flight.
    asm volatile("s_barrier" ::: "memory");
    if (p + kStages - 1 < npairs) pl.issue(p + kStages - 1);
    if (!has_rows) continue;

    const unsigned char* st = lds_buf + (p % kStages) * SG::kBytes;
    TileMeta mt[2];
    int delta[2];
    bool priv[2];
    pl.pair_meta(p, mt, delta, priv);

    // scores S^T[key 4g+j][row r] of both tiles, raw (unscaled)
    f32x4 s[2][RB];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      if (P::kRot && delta[x] != cur_delta) {
        pl.rotate(qr, raw, st, x, delta[x]);
        cur_delta = delta[x];
      }
      F8 kf[NC];
      const unsigned char* kt = st + SG::kK + x * SG::kTile + r * (DH * 2);
#pragma unroll
      for (int c = 0; c < NC; ++c)
        kf[c] = *reinterpret_cast<const F8*>(kt + (((4 * c + g) ^ (r % SG::kChunksPerRow)) << 4));
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[c], qr[b][c], z, 0, 0, 0);
        s[x][b] = z;
      }
    }
    // V^T operand of channel block n: slots 0..3 = tile 0 tokens 4g..4g+3,
    // slots 4..7 = tile 1 tokens 4g..4g+3 (the keys this lane's scores hold)
    F8 vv[NV];
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      const int off = (16 * n + r) * 32 + (((g >> 1) ^ ((r >> 3) & 1)) << 4) + ((g & 1) << 3);
      const F4 lo = *reinterpret_cast<const F4*>(st + SG::kV + off);
      const F4 hi = *reinterpret_cast<const F4*>(st + SG::kV + SG::kTile + off);
      vv[n] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }

    // Masking only where a slot can be invalid: partial or dropped tiles,
    // causal private tiles, ALiBi bias (wave-uniform test on the words).
    const bool full = KIND != kAlibi && (mt[0].mask & mt[1].mask) == 0xFFFFu && !priv[0] && !priv[1];
    if (!full) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int slot = 4 * g + j;
          const bool filled = (mt[x].mask >> slot) & 1u;
          const int kpos = mt[x].offset + slot;
#pragma unroll
          for (int b = 0; b < RB; ++b) {
            const bool ok = filled && (!priv[x] || kpos <= qp[b]);
            float v = s[x][b][j];
            if (KIND == kAlibi) v = fmaf(slope_raw[b], (float)(kpos - qp[b]), v);
            s[x][b][j] = ok ? v : -INFINITY;
          }
          // empty slots hold unwritten pool bytes: zero their V (p is 0 there)
          if (!filled) {
#pragma unroll
            for (int n = 0; n < NV; ++n) vv[n][4 * x + j] = (bf16)0.f;
          }
        }
      }
    }

    // Lazy rescale: the reference max m_run only moves (and acc, l are
    // rescaled) when some row's score exceeds it by more than 2^SLACK, so
    // every weight stays <= 2^SLACK; exact in real arithmetic, and the combine
    // uses the same reference.  Checked per lane on raw scores (scale > 0).
    float mx[RB];
    bool grow = false;
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      float m = fmaxf(s[0][b][0], s[0][b][1]);
      m = fmaxf(m, fmaxf(s[0][b][2], s[0][b][3]));
      m = fmaxf(m, fmaxf(s[1][b][0], s[1][b][1]));
      m = fmaxf(m, fmaxf(s[1][b][2], s[1][b][3]));
      mx[b] = m;
      grow = grow || (m > thr[b]);
    }
    if (__any(grow)) {
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const float m_new = fmaxf(m_run[b], xor_max16_32(mx[b]) * sl);
        const float alpha = (m_run[b] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[b] - m_new);
#pragma unroll
        for (int n = 0; n < NV; ++n) acc[b][n] *= alpha;
        lsum[b] *= alpha;
        m_run[b] = m_new;
        const bool none = m_new == -INFINITY;
        negm[b] = none ? 0.f : -m_new;
        thr[b] = none ? -INFINITY : (m_new + (float)LAZY_RESCALE_SLACK) / sl;
      }
    }

    // weights p = 2^(s * scale_log2 - m_run), row sums and P V on the MFMAs
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      F8 pf;
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int j = 0; j < 4; ++j) pf[4 * x + j] = (bf16)__builtin_amdgcn_exp2f(fmaf(s[x][b][j], sl, negm[b]));
      lsum[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf, lsum[b], 0, 0, 0);
#pragma unroll
      for (int n = 0; n < NV; ++n) acc[b][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv[n], pf, acc[b][n], 0, 0, 0);
    }
  }
  if (!has_rows) return;

  // O[row r][16n + 4g + j] = acc[b][n][j]: normalised output (one split) or an
  // unnormalised (m, l, acc) partial for the combine.
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int rho = (rb0 + b) * 16 + r;
    if (rho >= nrows) continue;
    const int orow = (q0 + rho / a.group) * a.hq + kvh * a.group + rho % a.group;
    const float l_tot = lsum[b][0];
    if (a.num_splits == 1) {
      const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
      bf16* o = reinterpret_cast<bf16*>(a.out) + (int64_t)orow * DH + 4 * g;
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        F4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = (bf16)(acc[b][n][j] * inv);
        *reinterpret_cast<F4*>(o + 16 * n) = w;
      }
    } else {
      const int64_t prow = (int64_t)split * a.rows_bound + orow;
      float* po = a.part_o + prow * DH + 4 * g;
#pragma unroll
      for (int n = 0; n < NV; ++n) *reinterpret_cast<f32x4*>(po + 16 * n) = acc[b][n];
      if (g == 0) {
        a.part_ml[prow * 2 + 0] = m_run[b];
        a.part_ml[prow * 2 + 1] = l_tot;
      }
    }
  }
}

namespace {

template <int DH, int KIND, bool DEFER, int RB, int NW>
hipError_t launch_rb(const AttnArgs& a, int row_tiles, int splits, int num_reqs, int hkv, hipStream_t st) {
  constexpr bool rot = (KIND != kAlibi) && DEFER;
  const size_t lds = (size_t)kStages * StageGeom<DH, rot, NW>::kBytes + (size_t)NW * RB * (DH / 32) * 64 * 16;
  static bool attr_set = false;  // the ring needs more than the default 64 KiB of dynamic LDS
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&prefill_lds_kernel<DH, KIND, DEFER, RB, NW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid((unsigned)(row_tiles * splits), (unsigned)hkv, (unsigned)num_reqs);
  hipLaunchKernelGGL((prefill_lds_kernel<DH, KIND, DEFER, RB, NW>), grid, dim3(64 * NW), lds, st, a);
  return hipGetLastError();
}

// rows per workgroup = 16 x rb x 4 (the host plan's row tile)
template <int DH, int KIND, bool DEFER>
hipError_t launch_kind(const AttnArgs& a, int rb, int row_tiles, int splits, int num_reqs, int hkv, hipStream_t st) {
  constexpr int NW = LAZY_PREFILL_LDS_WAVES;
  static_assert(NW == 4 || NW == 8, "waves per workgroup");
  if (NW == 8)
    return rb == 4 ? launch_rb<DH, KIND, DEFER, 2, NW>(a, row_tiles, splits, num_reqs, hkv, st)
                   : launch_rb<DH, KIND, DEFER, 1, NW>(a, row_tiles, splits, num_reqs, hkv, st);
  return rb == 4 ? launch_rb<DH, KIND, DEFER, 4, 4>(a, row_tiles, splits, num_reqs, hkv, st)
                 : launch_rb<DH, KIND, DEFER, 2, 4>(a, row_tiles, splits, num_reqs, hkv, st);
}

template <int DH>
hipError_t launch_dh(const AttnArgs& a, int kind, bool defer, int rb, int row_tiles, int splits, int num_reqs,
                     int hkv, hipStream_t st) {
  switch (kind) {
    case kHalf:
      return defer ? launch_kind<DH, kHalf, true>(a, rb, row_tiles, splits, num_reqs, hkv, st)
                   : launch_kind<DH, kHalf, false>(a, rb, row_tiles, splits, num_reqs, hkv, st);
    case kInter:
      return defer ? launch_kind<DH, kInter, true>(a, rb, row_tiles, splits, num_reqs, hkv, st)
                   : launch_kind<DH, kInter, false>(a, rb, row_tiles, splits, num_reqs, hkv, st);
    default:
      return launch_kind<DH, kAlibi, false>(a, rb, row_tiles, splits, num_reqs, hkv, st);
  }
}

}  // namespace

hipError_t launch_prefill_lds(const AttnArgs& a, int kind, bool defer, int head_dim, int rb, int row_tiles,
                              int splits, int num_reqs, int hkv, hipStream_t st) {
  if (rb != 2 && rb != 4) return hipErrorNotSupported;
  if (kind != kAlibi && defer && a.cos_sin == nullptr) return hipErrorNotSupported;  // rows come from the table
  if (head_dim == 128) return launch_dh<128>(a, kind, defer, rb, row_tiles, splits, num_reqs, hkv, st);
  if (head_dim == 64) return launch_dh<64>(a, kind, defer, rb, row_tiles, splits, num_reqs, hkv, st);
  return hipErrorNotSupported;
}

}  // namespace lazy
