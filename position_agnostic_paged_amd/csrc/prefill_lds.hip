// LDS-staged prefill over a position-agnostic paged cache (bf16, gfx950).
//
// Same computation as the per-wave prefill (LazyAttention notes,
// papernotes.org, "Key designs": compute-bound prefill with the document
// offset applied inside the fused kernel), organised for CDNA4:
//
//   * a workgroup = 4 waves x RB blocks of 16 GQA-packed query rows of one
//     (request, KV head); all four waves consume the same tile pairs;
//   * each tile pair (K 2 x 16 x dh, V 2 x dh x 16, plus the two cos/sin
//     rows of the pair's document offsets) is copied once per workgroup
//     from HBM into LDS with direct global->LDS loads (no registers), into a
//     ring of kStages buffers, so kStages-1 pairs are in flight while one is
//     consumed by the MFMAs;
//   * LDS rows are XOR-swizzled at 16-byte granularity so the per-lane
//     fragment reads (16 B of a K row, 8 B of a V channel row) are free of
//     bank conflicts;
//   * the query is re-rotated by -Delta once per document from the raw
//     query kept in registers and the cos/sin row in the stage, so the loop
//     issues no global load besides the stage copies (keeping the counted
//     waits on the copies exact).
#include "attn_common.hpp"

namespace lazy {

constexpr int kLdsWaves = 4;   // waves per workgroup
constexpr int kStages = 4;     // LDS ring of tile pairs

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

template <int DH, bool ROT>
struct StageGeom {
  static constexpr int kTile = kBlock * DH * 2;          // bytes of one 16 x dh bf16 tile
  static constexpr int kChunksPerRow = DH / 8;           // 16-byte chunks in a K row
  static constexpr int kK = 0;                           // two K tiles
  static constexpr int kV = 2 * kTile;                   // two V tiles
  static constexpr int kCS = 4 * kTile;                  // two cos/sin rows (fp32 [dh])
  static constexpr int kBytes = 4 * kTile + (ROT ? 2 * DH * 4 : 0);
  static constexpr int kKVCopies = (2 * kTile) / (kLdsWaves * 64 * 16);  // 16-B copies per thread for K (same for V)
  static constexpr int kLoads = 2 * kKVCopies + (ROT ? 1 : 0);         // copies per thread per stage
  static_assert(kKVCopies >= 1, "tile pair smaller than one copy round");
};

typedef const __attribute__((address_space(4))) uint64_t* const_words;

// Per-workgroup state and steps of the staged prefill (device functions, not
// lambdas: the kernel template must also instantiate on the host side).
template <int DH, int KIND, bool DEFER, int RB>
struct LdsPrefill {
  using W = WaveAttn<bf16, DH, KIND, DEFER, true, RB, 1>;
  using F8 = typename W::F8;
  using F4 = typename W::F4;
  static constexpr int NC = DH / 32;
  static constexpr int NV = DH / 16;
  static constexpr bool kRot = W::kRot;
  using SG = StageGeom<DH, kRot>;

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
      if (mt[x].block >= a.num_blocks || mt[x].block < 0) {
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

  // copy pair p into stage buffer p % kStages (every thread issues SG::kLoads copies)
  __device__ __forceinline__ void issue(int p) const {
    TileMeta mt[2];
    int delta[2];
    bool priv[2];
    pair_meta(p, mt, delta, priv);
    unsigned char* st = lds + (p % kStages) * SG::kBytes;
    const bf16* kc = reinterpret_cast<const bf16*>(a.k_cache);
    const bf16* vc = reinterpret_cast<const bf16*>(a.v_cache);
#pragma unroll
    for (int i = 0; i < SG::kKVCopies; ++i) {
      const int ci = i * kLdsWaves * 64 + tid;  // 16-B chunk of the K pair
      const int x = ci / (SG::kTile / 16);
      const int cc = ci % (SG::kTile / 16);
      const int row = cc / SG::kChunksPerRow, pos = cc % SG::kChunksPerRow;
      const int q = pos ^ (row % SG::kChunksPerRow);
      const int blk = x ? mt[1].block : mt[0].block;
      const bf16* src = kc + ((int64_t)blk * a.hkv + kvh) * (kBlock * DH) + row * DH + q * 8;
      __builtin_amdgcn_global_load_lds(src, st + SG::kK + (i * kLdsWaves + wave) * 64 * 16, 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < SG::kKVCopies; ++i) {
      const int ci = i * kLdsWaves * 64 + tid;  // 16-B chunk of the V pair (rows of 16 tokens = 32 B)
      const int x = ci / (SG::kTile / 16);
      const int cc = ci % (SG::kTile / 16);
      const int row = cc >> 1, pos = cc & 1;
      const int q = pos ^ ((row >> 3) & 1);
      const int blk = x ? mt[1].block : mt[0].block;
      const bf16* src = vc + ((int64_t)blk * a.hkv + kvh) * (kBlock * DH) + row * kBlock + q * 8;
      __builtin_amdgcn_global_load_lds(src, st + SG::kV + (i * kLdsWaves + wave) * 64 * 16, 16, 0, 0);
    }
    if (kRot) {
      // the two cos/sin rows: DH/4 chunks each; wave w copies its share (lane-masked)
      constexpr int kCsChunks = 2 * (DH / 4);
      constexpr int kPerWave = kCsChunks / kLdsWaves;
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
  __device__ __forceinline__ void rotate(W& w, const unsigned char* raw, const unsigned char* st, int x,
                                         int delta) const {
    if (delta == 0) {
#pragma unroll
      for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int c = 0; c < NC; ++c) w.qr[0][b][c] = raw_at(raw, b, c);
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
            w.qr[0][b][c][t] = (bf16)(x1 * cs + x2 * sn);
            w.qr[0][b][c + NC / 2][t] = (bf16)(x2 * cs - x1 * sn);
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
            w.qr[0][b][c][2 * u] = (bf16)(x1 * c0[u] + x2 * s0[u]);
            w.qr[0][b][c][2 * u + 1] = (bf16)(x2 * c0[u] - x1 * s0[u]);
          }
        }
      }
    }
  }
};

template <int DH, int KIND, bool DEFER, int RB>
__global__ __launch_bounds__(64 * kLdsWaves, 1) void prefill_lds_kernel(AttnArgs a) {
  using P = LdsPrefill<DH, KIND, DEFER, RB>;
  using W = typename P::W;
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
  if (row_tile * kLdsWaves * RB * 16 >= nrows) return;
  if (!split_range(nt, a.chunk, a.num_splits, split, sb, se)) return;
  const int npairs = (se - sb + 1) >> 1;
  const int rb0 = (row_tile * kLdsWaves + wave) * RB;
  const bool has_rows = rb0 * 16 < nrows;  // wave-uniform: waves without rows still copy tiles

  P pl{a, lds_buf, tid, lane, wave, r, g, kvh, sb, se, a.ctx_tiles[req], (const_words)(a.tiles + t0)};

  // a wave without rows builds its (unused) state from the first rows, which exist
  W w(a, lane, kvh, req, q0, nrows, has_rows ? rb0 : 0, a.q_pos[req]);
  // the query at its global position, the source of every re-rotation, is
  // parked in this wave's LDS area (fragment order, 16 B per lane)
  unsigned char* raw = lds_buf + kStages * SG::kBytes + wave * (RB * NC * 64 * 16);
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int c = 0; c < NC; ++c) *reinterpret_cast<F8*>(raw + ((b * NC + c) * 64 + lane) * 16) = w.qr[0][b][c];
  int cur_delta = 0;

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
    typename W::Pair pr;
    pl.pair_meta(p, pr.mt, pr.delta, pr.priv);
    f32x4 s[2][RB];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      if (P::kRot && pr.delta[x] != cur_delta) {
        pl.rotate(w, raw, st, x, pr.delta[x]);
        cur_delta = pr.delta[x];
      }
      F8 kf[NC];
      const unsigned char* kt = st + SG::kK + x * SG::kTile + r * (DH * 2);
#pragma unroll
      for (int c = 0; c < NC; ++c)
        kf[c] = *reinterpret_cast<const F8*>(kt + (((4 * c + g) ^ (r % SG::kChunksPerRow)) << 4));
      w.scores(kf, 0, s[x]);
    }
    F4 vf[2][NV];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const unsigned char* vt = st + SG::kV + x * SG::kTile;
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        const int row = 16 * n + r;
        vf[x][n] = *reinterpret_cast<const F4*>(vt + row * 32 + (((g >> 1) ^ ((r >> 3) & 1)) << 4) + ((g & 1) << 3));
      }
    }
    w.softmax_pv(pr, vf, s);
  }
  if (has_rows) w.finalize(split);
}

namespace {

template <int DH, int KIND, bool DEFER, int RB>
hipError_t launch_rb(const AttnArgs& a, int row_tiles, int splits, int num_reqs, int hkv, hipStream_t st) {
  constexpr bool rot = (KIND != kAlibi) && DEFER;
  const size_t lds = (size_t)kStages * StageGeom<DH, rot>::kBytes + (size_t)kLdsWaves * RB * (DH / 32) * 64 * 16;
  static bool attr_set = false;  // the ring needs more than the default 64 KiB of dynamic LDS
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_lds_kernel<DH, KIND, DEFER, RB>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid((unsigned)(row_tiles * splits), (unsigned)hkv, (unsigned)num_reqs);
  hipLaunchKernelGGL((prefill_lds_kernel<DH, KIND, DEFER, RB>), grid, dim3(64 * kLdsWaves), lds, st, a);
  return hipGetLastError();
}

template <int DH, int KIND, bool DEFER>
hipError_t launch_kind(const AttnArgs& a, int rb, int row_tiles, int splits, int num_reqs, int hkv, hipStream_t st) {
  return rb == 4 ? launch_rb<DH, KIND, DEFER, 4>(a, row_tiles, splits, num_reqs, hkv, st)
                 : launch_rb<DH, KIND, DEFER, 2>(a, row_tiles, splits, num_reqs, hkv, st);
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
