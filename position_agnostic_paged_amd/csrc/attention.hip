// Fused paged attention over a position-agnostic KV cache with the document
// offset applied inside the kernel (prefill and decode), plus the split-K
// log-sum-exp combine.
//
// What is computed (LazyAttention notes, papernotes.org, "Method: overall
// framework" and "Key designs"; gist.science summary, "Implementazione
// Tecnica"): for every query row, softmax(scale * q . k' + bias) V over the
// request's tiles, where k' is the key at its global position.  Cached
// document keys are stored rotated at document-local positions, so
// k' = R_Delta k_cached; the kernel applies the equivalent single relative
// rotation to the query, q' = R_{-Delta} q, because (R_{-D} q) . k =
// q . (R_D k) exactly (RoPE relativity, notes "Background and motivation").
//
// MI355X design (differs from the pages' Triton kernels, see the design doc):
//   * One kernel for prefill and decode.  Query rows are GQA-packed: the G
//     query heads of a KV head (x the query tokens in prefill) form the
//     16-wide column blocks of the MFMA products, so a K/V tile is read once
//     for all G heads (notes, "Generality": GQA/MQA need no change).
//   * S^T = K Q'^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16: the K
//     cache is token-major and the V cache channel-major inside a block, so
//     both operands load straight from HBM with 16-byte (K) / 8-byte (V)
//     coalesced loads, no LDS staging, and the score layout out of the first
//     product is exactly the B operand of the second.
//   * The query is re-rotated only when the tile's Delta changes, i.e. once
//     per document, in prefill and decode alike (the notes' decode rule;
//     in prefill it replaces the per-tile K rotation of the pages' kernel:
//     on gfx950 a VALU rotation of every K tile costs more issue slots than
//     the tile's MFMA work, while one query rotation per document is ~1/L of
//     that).  Each lane owns whole rotation pairs, so rotation is lane-local.
//   * The tile word (block, offset, mask) is one wave-uniform 8-byte load,
//     split with shifts; no block-table, offset or mask arrays are read.
//   * Split-K over tiles: every (request, KV head, row tile, split) wave
//     writes (m, l, acc) partials when more than one split is used.
//   * Masked slots are selected to -inf (never multiplied) and their V
//     values to 0, so garbage in unused slots of partial blocks cannot leak.
#include <math.h>

#include <algorithm>

#include "lazy_device.hpp"
#include "lazy_host.hpp"

namespace lazy {

struct AttnArgs {
  const void* k_cache;
  const void* v_cache;
  int64_t num_blocks;
  const uint64_t* tiles;
  const int32_t* tile_start;
  const int32_t* ctx_tiles;
  const void* q;
  const int32_t* q_start;  // prefill: row range per request; decode: unused (row r = request r)
  const int32_t* q_pos;    // prefill: position of the first query row; decode: query position
  const float* cos_sin;    // [max_pos][DH] or NULL (on-the-fly from inv_freq)
  const double* inv_freq;
  int32_t max_pos;
  const float* slopes;
  float scale_log2;  // softmax_scale * log2(e)
  void* out;
  float* part_o;  // [splits][rows_bound][DH]
  float* part_ml;  // [splits][rows_bound][2]
  int32_t num_splits;
  int32_t splits_per_wg;  // waves along splits inside a workgroup
  int32_t hq, hkv, group;
  int32_t rows_bound;  // partial row stride: (max query rows) * hq
  int32_t max_q_len;   // prefill: rows per request covered by the grid
};

enum { kHalf = LAZY_ROPE_HALF, kInter = LAZY_ROPE_INTERLEAVED, kAlibi = LAZY_ALIBI };

// cos/sin of Delta * theta_k for the pair indices this lane owns.
// Half-split: lane (g) owns pairs k = 32c + 8g + t (c < DH/64, t < 8).
// Interleaved: lane owns pairs k = 16c + 4g + u (c < DH/32, u < 4).
template <int DH, int KIND>
struct RotCoef {
  static constexpr int N = (KIND == kHalf) ? (DH / 64) * 8 : (DH / 32) * 4;
  float c[N], s[N];

  __device__ __forceinline__ void load(const AttnArgs& a, int delta, int g) {
    if (a.cos_sin != nullptr) {
      const float* row = a.cos_sin + (int64_t)delta * DH;
      if (KIND == kHalf) {
#pragma unroll
        for (int cc = 0; cc < DH / 64; ++cc) {
          const f32x4* pc = reinterpret_cast<const f32x4*>(row + 32 * cc + 8 * g);
          const f32x4* ps = reinterpret_cast<const f32x4*>(row + DH / 2 + 32 * cc + 8 * g);
          f32x4 c0 = pc[0], c1 = pc[1], s0 = ps[0], s1 = ps[1];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            c[cc * 8 + t] = c0[t];
            c[cc * 8 + 4 + t] = c1[t];
            s[cc * 8 + t] = s0[t];
            s[cc * 8 + 4 + t] = s1[t];
          }
        }
      } else {
#pragma unroll
        for (int cc = 0; cc < DH / 32; ++cc) {
          f32x4 c0 = *reinterpret_cast<const f32x4*>(row + 16 * cc + 4 * g);
          f32x4 s0 = *reinterpret_cast<const f32x4*>(row + DH / 2 + 16 * cc + 4 * g);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            c[cc * 4 + u] = c0[u];
            s[cc * 4 + u] = s0[u];
          }
        }
      }
    } else {
      // on-the-fly coefficients (no table reads)
#pragma unroll
      for (int i = 0; i < N; ++i) {
        int k;
        if (KIND == kHalf)
          k = 32 * (i / 8) + 8 * g + (i % 8);
        else
          k = 16 * (i / 4) + 4 * g + (i % 4);
        sincos_reduced(delta, a.inv_freq[k], &s[i], &c[i]);
      }
    }
  }
};

// q' = R_{-delta} q for the RB row blocks of this wave (lane-local pairs).
template <typename T, int DH, int KIND, int RB>
__device__ __forceinline__ void rotate_query(typename Elem<T>::Frag8 (&qr)[RB][DH / 32], const T* const (&qptr)[RB],
                                             const AttnArgs& a, int delta, int g, int active_blocks) {
  using E = Elem<T>;
  using F8 = typename E::Frag8;
  constexpr int NC = DH / 32;
  F8 raw[RB][NC];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    if (b < active_blocks) {
#pragma unroll
      for (int c = 0; c < NC; ++c) raw[b][c] = load8<T>(qptr[b] + 32 * c + 8 * g);
    }
  }
  if (KIND == kAlibi || delta == 0) {
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int c = 0; c < NC; ++c) qr[b][c] = raw[b][c];
    return;
  }
  RotCoef<DH, KIND> rc;
  rc.load(a, delta, g);
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    if (b >= active_blocks) continue;
    if (KIND == kHalf) {
#pragma unroll
      for (int c = 0; c < NC / 2; ++c) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float x1 = E::to_f(raw[b][c][t]);
          const float x2 = E::to_f(raw[b][c + NC / 2][t]);
          const float cs = rc.c[c * 8 + t], sn = rc.s[c * 8 + t];
          qr[b][c][t] = E::from_f(x1 * cs + x2 * sn);           // rotation by -delta
          qr[b][c + NC / 2][t] = E::from_f(x2 * cs - x1 * sn);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float x1 = E::to_f(raw[b][c][2 * u]);
          const float x2 = E::to_f(raw[b][c][2 * u + 1]);
          const float cs = rc.c[c * 4 + u], sn = rc.s[c * 4 + u];
          qr[b][c][2 * u] = E::from_f(x1 * cs + x2 * sn);
          qr[b][c][2 * u + 1] = E::from_f(x2 * cs - x1 * sn);
        }
      }
    }
  }
}

// One wave = RB blocks of 16 query rows x one split of the request's tiles.
// Workgroup = WR waves along rows x WT waves along splits.
template <typename T, int DH, int KIND, bool DEFER, bool PREFILL, int RB, int WR, int WT>
__global__ __launch_bounds__(64 * WR * WT) void attn_kernel(AttnArgs a) {
  using E = Elem<T>;
  using F8 = typename E::Frag8;
  using F4 = typename E::Frag4;
  constexpr int NC = DH / 32;  // contraction chunks of QK^T
  constexpr int NV = DH / 16;  // 16-channel blocks of the output

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wr = wave % WR;
  const int wt = wave / WR;
  const int r = lane & 15;
  const int g = lane >> 4;

  const int req = blockIdx.z;
  const int kvh = blockIdx.y;
  const int wg_per_rt = a.num_splits / WT;
  const int row_tile = blockIdx.x / wg_per_rt;
  const int split = (blockIdx.x % wg_per_rt) * WT + wt;

  int q0, nq;
  if (PREFILL) {
    q0 = a.q_start[req];
    nq = a.q_start[req + 1] - q0;
    // never address query rows beyond what the grid and workspace were sized for
    nq = min(nq, a.max_q_len);
    nq = max(0, min(nq, a.rows_bound / a.hq - q0));
  } else {
    q0 = req;
    nq = 1;
  }
  const int nrows = nq * a.group;
  const int rb0 = (row_tile * WR + wr) * RB;  // first 16-row block of this wave
  if (rb0 * 16 >= nrows) return;              // no work for this wave (no barriers follow)
  const int active_blocks = min(RB, (nrows - rb0 * 16 + 15) / 16);

  const int qpos0 = a.q_pos[req];
  const int t0 = a.tile_start[req];
  const int nt = a.tile_start[req + 1] - t0;
  const int nctx = a.ctx_tiles[req];

  // this split's tile range (pairs of tiles; the last pair may be half empty)
  int chunk = (nt + a.num_splits - 1) / a.num_splits;
  chunk = (chunk + 1) & ~1;
  const int sb = min(nt, split * chunk);
  const int se = min(nt, sb + chunk);
  const int npairs = (se - sb + 1) >> 1;

  // per-lane row bookkeeping for each row block
  const T* qptr[RB];
  int qp[RB];
  int orow[RB];
  bool rvalid[RB];
  float slope2[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int rho = (rb0 + b) * 16 + r;
    rvalid[b] = rho < nrows;
    const int rr = rvalid[b] ? rho : 0;
    const int qi = rr / a.group;
    const int head = kvh * a.group + rr % a.group;
    qptr[b] = reinterpret_cast<const T*>(a.q) + ((int64_t)(q0 + qi) * a.hq + head) * DH;
    qp[b] = qpos0 + qi;
    orow[b] = (q0 + qi) * a.hq + head;
    slope2[b] = (KIND == kAlibi) ? a.slopes[head] * kLog2e : 0.f;
  }

  // Rotated query per tile slot of a pair (x = 0: even tile, 1: odd tile).
  // Keeping one set per slot lets every re-rotation happen at the top of a
  // pair iteration, before its K/V fragments are loaded, so the rotation's
  // registers never overlap theirs; a document costs at most two rotations.
  constexpr bool kRot = (KIND != kAlibi) && DEFER;
  constexpr int NQ = kRot ? 2 : 1;
  F8 qr[NQ][RB][NC];
  rotate_query<T, DH, KIND, RB>(qr[0], qptr, a, 0, g, active_blocks);
  if (NQ > 1) {
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int c = 0; c < NC; ++c) qr[NQ - 1][b][c] = qr[0][b][c];
  }
  int cur_delta[2] = {0, 0};

  f32x4 acc[RB][NV];
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    m_run[b] = -INFINITY;
    l_run[b] = 0.f;
#pragma unroll
    for (int n = 0; n < NV; ++n) acc[b][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const T* kc = reinterpret_cast<const T*>(a.k_cache);
  const T* vc = reinterpret_cast<const T*>(a.v_cache);
  const int64_t head_stride = (int64_t)kBlock * DH;

  for (int p = 0; p < npairs; ++p) {
    const int ia = sb + 2 * p;  // tile index within the request
    const int ib = ia + 1;
    TileMeta mt[2];
    mt[0] = unpack_word(a.tiles[t0 + ia]);
    if (ib < se) {
      mt[1] = unpack_word(a.tiles[t0 + ib]);
    } else {
      mt[1] = mt[0];
      mt[1].mask = 0u;
    }
    int delta[2];
    bool priv[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int ti = ia + x;
      priv[x] = ti >= nctx;
      if (mt[x].block >= a.num_blocks || mt[x].block < 0) {  // never dereference outside the pool
        mt[x].block = 0;
        mt[x].mask = 0u;
      }
      delta[x] = (kRot && !priv[x]) ? mt[x].offset : 0;
      if (delta[x] >= a.max_pos && a.cos_sin != nullptr) {  // outside the table: drop the tile
        mt[x].mask = 0u;
        delta[x] = cur_delta[x];
      }
      // single relative rotation of the query when the document changes
      if (kRot && delta[x] != cur_delta[x]) {
        rotate_query<T, DH, KIND, RB>(qr[x * (NQ - 1)], qptr, a, delta[x], g, active_blocks);
        cur_delta[x] = delta[x];
      }
    }

    // issue all K and V loads of the pair
    F8 kf[2][NC];
    F4 vf[2][NV];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int64_t base = ((int64_t)mt[x].block * a.hkv + kvh) * head_stride;
      const T* kp = kc + base + r * DH + 8 * g;
      const T* vp = vc + base + r * kBlock + 4 * g;
#pragma unroll
      for (int c = 0; c < NC; ++c) kf[x][c] = load8<T>(kp + 32 * c);
#pragma unroll
      for (int n = 0; n < NV; ++n) vf[x][n] = load4<T>(vp + n * 16 * kBlock);
    }

    // scores S^T[key 4g+j][row r] for both tiles
    f32x4 s[2][RB];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        if (b < active_blocks) {
#pragma unroll
          for (int c = 0; c < NC; ++c) z = E::mma(kf[x][c], qr[x * (NQ - 1)][b][c], z);
        }
        s[x][b] = z;
      }
    }

    // zero V of empty slots (partial blocks, dropped tiles)
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      if (mt[x].mask != 0xFFFFu) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool ok = (mt[x].mask >> (4 * g + j)) & 1u;
#pragma unroll
          for (int n = 0; n < NV; ++n) vf[x][n][j] = ok ? vf[x][n][j] : E::from_f(0.f);
        }
      }
    }

#pragma unroll
    for (int b = 0; b < RB; ++b) {
      if (b >= active_blocks) continue;
      float sv[2][4];
      float mx = -INFINITY;
#pragma unroll
      for (int x = 0; x < 2; ++x) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int slot = 4 * g + j;
          bool ok = (mt[x].mask >> slot) & 1u;
          const int kpos = mt[x].offset + slot;
          if (PREFILL && priv[x]) ok = ok && (kpos <= qp[b]);
          float v = s[x][b][j] * a.scale_log2;
          if (KIND == kAlibi) v += slope2[b] * (float)(kpos - qp[b]);
          v = ok ? v : -INFINITY;
          sv[x][j] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = xor_max16_32(mx);
      const float m_new = fmaxf(m_run[b], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[b] - m_use);
      F8 pf;
      float psum = 0.f;
#pragma unroll
      for (int x = 0; x < 2; ++x) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float pj = __builtin_amdgcn_exp2f(sv[x][j] - m_use);
          psum += pj;
          pf[4 * x + j] = E::from_f(pj);
        }
      }
      l_run[b] = l_run[b] * alpha + psum;
      m_run[b] = m_new;
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        acc[b][n] *= alpha;
        F8 v8;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v8[j] = vf[0][n][j];
          v8[4 + j] = vf[1][n][j];
        }
        acc[b][n] = E::mma(v8, pf, acc[b][n]);
      }
    }
  }

  // finalize: O[row r][16n + 4g + j] = acc[b][n][j]
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    if (b >= active_blocks) continue;
    const float l_tot = xor_sum16_32(l_run[b]);
    if (!rvalid[b]) continue;
    if (a.num_splits == 1) {
      const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
      T* o = reinterpret_cast<T*>(a.out) + (int64_t)orow[b] * DH + 4 * g;
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        F4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = E::from_f(acc[b][n][j] * inv);
        *reinterpret_cast<F4*>(o + 16 * n) = w;
      }
    } else {
      const int64_t prow = (int64_t)split * a.rows_bound + orow[b];
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

// Split-K combine (flash-decoding): for every output row,
//   M = max_s m_s,  out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
// Splits that saw no visible key carry m = -inf and contribute nothing.
template <typename T, int DH>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml, T* __restrict__ out,
                                                      const int32_t* __restrict__ q_start, int32_t num_reqs,
                                                      int32_t hq, int32_t rows_bound, int32_t num_splits,
                                                      int32_t rows_fixed) {
  constexpr int TPR = DH / 4;  // threads per row, 4 channels each
  const int row = blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int c4 = (threadIdx.x % TPR) * 4;
  const int rows = min(rows_bound, (q_start != nullptr) ? q_start[num_reqs] * hq : rows_fixed);
  if (row >= rows) return;
  float M = -INFINITY;
  for (int s = 0; s < num_splits; ++s) M = fmaxf(M, part_ml[((int64_t)s * rows_bound + row) * 2]);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  float L = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < num_splits; ++s) {
    const int64_t pr = (int64_t)s * rows_bound + row;
    const float w = __builtin_amdgcn_exp2f(part_ml[pr * 2] - Mu);
    L += w * part_ml[pr * 2 + 1];
    const f32x4 v = *reinterpret_cast<const f32x4*>(part_o + pr * DH + c4);
    o += w * v;
  }
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
  using F4 = typename Elem<T>::Frag4;
  F4 w4;
#pragma unroll
  for (int j = 0; j < 4; ++j) w4[j] = Elem<T>::from_f(o[j] * inv);
  *reinterpret_cast<F4*>(out + (int64_t)row * DH + c4) = w4;
}

__global__ void debug_unpack_kernel(const uint64_t* w, int64_t n, int32_t* blk, int32_t* off, int32_t* msk) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const TileMeta t = unpack_word(w[i]);
  blk[i] = t.block;
  off[i] = t.offset;
  msk[i] = (int32_t)t.mask;
}

// ------------------------------------------------------------------ host side

namespace {

constexpr int kPrefillRB = 2, kPrefillWR = 4;  // 128 query rows per workgroup
constexpr int kDecodeWT = 4;                   // 4 waves = 4 splits per workgroup

int decode_rb(int group) { return group <= 16 ? 1 : group <= 32 ? 2 : group <= 64 ? 4 : 8; }

struct Plan {
  int rb, wr, wt;
  int row_tiles;
  int splits;
  int rows_bound;
};

Plan make_plan(const lazy_geom* g, int num_reqs, int max_q_len, int max_tiles, bool prefill) {
  Plan p;
  const int group = g->num_q_heads / g->num_kv_heads;
  if (prefill) {
    p.rb = kPrefillRB;
    p.wr = kPrefillWR;
    p.wt = 1;
    const int rows = max_q_len * group;
    p.row_tiles = (rows + 16 * p.rb * p.wr - 1) / (16 * p.rb * p.wr);
    const long units = (long)num_reqs * g->num_kv_heads * p.row_tiles;
    int s = (int)((512 + units - 1) / units);
    s = std::min(s, std::max(1, max_tiles / 16));
    p.splits = std::max(1, std::min(s, 64));
    p.rows_bound = max_q_len * num_reqs * g->num_q_heads;
  } else {
    p.rb = decode_rb(group);
    p.wr = 1;
    p.wt = kDecodeWT;
    p.row_tiles = 1;
    const long units = (long)num_reqs * g->num_kv_heads;
    int s = (int)((2048 * p.wt + units - 1) / units);
    s = std::min(s, std::max(1, max_tiles / 32));
    s = std::max(1, std::min(s, 256));
    s = (s + p.wt - 1) / p.wt * p.wt;  // whole workgroups
    p.splits = s;
    p.rows_bound = num_reqs * g->num_q_heads;
  }
  return p;
}

size_t ws_bytes_for(const lazy_geom* g, const Plan& p) {
  if (p.splits == 1) return 0;
  const size_t per = (size_t)g->head_dim + 2;
  return (size_t)p.splits * (size_t)p.rows_bound * per * sizeof(float) + 256;
}

template <typename T, int DH, int KIND, bool DEFER, bool PREFILL, int RB, int WR, int WT>
hipError_t launch_attn(const AttnArgs& a, const Plan& p, int num_reqs, int hkv, hipStream_t st) {
  dim3 grid((unsigned)(p.row_tiles * (p.splits / WT)), (unsigned)hkv, (unsigned)num_reqs);
  dim3 block(64 * WR * WT);
  hipLaunchKernelGGL((attn_kernel<T, DH, KIND, DEFER, PREFILL, RB, WR, WT>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <typename T, int DH, int KIND, bool DEFER, bool PREFILL>
hipError_t dispatch_rb(const AttnArgs& a, const Plan& p, int num_reqs, int hkv, hipStream_t st) {
  if (PREFILL) return launch_attn<T, DH, KIND, DEFER, true, kPrefillRB, kPrefillWR, 1>(a, p, num_reqs, hkv, st);
  switch (p.rb) {
    case 1:
      return launch_attn<T, DH, KIND, DEFER, false, 1, 1, kDecodeWT>(a, p, num_reqs, hkv, st);
    case 2:
      return launch_attn<T, DH, KIND, DEFER, false, 2, 1, kDecodeWT>(a, p, num_reqs, hkv, st);
    case 4:
      return launch_attn<T, DH, KIND, DEFER, false, 4, 1, kDecodeWT>(a, p, num_reqs, hkv, st);
    default:
      return launch_attn<T, DH, KIND, DEFER, false, 8, 1, kDecodeWT>(a, p, num_reqs, hkv, st);
  }
}

template <typename T, int DH, bool PREFILL>
hipError_t dispatch_kind(int kind, bool defer, const AttnArgs& a, const Plan& p, int num_reqs, int hkv,
                         hipStream_t st) {
  switch (kind) {
    case kHalf:
      return defer ? dispatch_rb<T, DH, kHalf, true, PREFILL>(a, p, num_reqs, hkv, st)
                   : dispatch_rb<T, DH, kHalf, false, PREFILL>(a, p, num_reqs, hkv, st);
    case kInter:
      return defer ? dispatch_rb<T, DH, kInter, true, PREFILL>(a, p, num_reqs, hkv, st)
                   : dispatch_rb<T, DH, kInter, false, PREFILL>(a, p, num_reqs, hkv, st);
    default:
      return dispatch_rb<T, DH, kAlibi, false, PREFILL>(a, p, num_reqs, hkv, st);
  }
}

template <typename T, int DH>
hipError_t launch_combine(const AttnArgs& a, const Plan& p, const int32_t* q_start, int num_reqs, int rows_fixed,
                          hipStream_t st) {
  constexpr int rows_per_block = 256 / (DH / 4);
  const int rows = p.rows_bound;
  dim3 grid((unsigned)((rows + rows_per_block - 1) / rows_per_block));
  hipLaunchKernelGGL((combine_kernel<T, DH>), grid, dim3(256), 0, st, a.part_o, a.part_ml,
                     reinterpret_cast<T*>(a.out), q_start, num_reqs, a.hq, p.rows_bound, p.splits, rows_fixed);
  return hipGetLastError();
}

template <bool PREFILL>
hipError_t run(const lazy_geom* g, const lazy_pos_desc* pd, AttnArgs& a, const Plan& p, int num_reqs,
               const int32_t* q_start, hipStream_t st) {
  const bool defer = !(pd->flags & LAZY_FLAG_PREROTATED);
  const int hkv = g->num_kv_heads;
  hipError_t e;
  if (g->dtype == LAZY_BF16) {
    e = (g->head_dim == 128) ? dispatch_kind<bf16, 128, PREFILL>(pd->kind, defer, a, p, num_reqs, hkv, st)
                             : dispatch_kind<bf16, 64, PREFILL>(pd->kind, defer, a, p, num_reqs, hkv, st);
  } else {
    e = (g->head_dim == 128) ? dispatch_kind<float, 128, PREFILL>(pd->kind, defer, a, p, num_reqs, hkv, st)
                             : dispatch_kind<float, 64, PREFILL>(pd->kind, defer, a, p, num_reqs, hkv, st);
  }
  if (e != hipSuccess || p.splits == 1) return e;
  const int rows_fixed = PREFILL ? 0 : num_reqs * g->num_q_heads;
  const int32_t* qs = PREFILL ? q_start : nullptr;
  if (g->dtype == LAZY_BF16)
    return (g->head_dim == 128) ? launch_combine<bf16, 128>(a, p, qs, num_reqs, rows_fixed, st)
                                : launch_combine<bf16, 64>(a, p, qs, num_reqs, rows_fixed, st);
  return (g->head_dim == 128) ? launch_combine<float, 128>(a, p, qs, num_reqs, rows_fixed, st)
                              : launch_combine<float, 64>(a, p, qs, num_reqs, rows_fixed, st);
}

lazy_status common_checks(const lazy_geom* g, const lazy_pos_desc* pd, const void* kc, const void* vc,
                          int64_t num_blocks, const uint64_t* tiles, const int32_t* tile_start,
                          const int32_t* ctx_tiles, const void* q, const int32_t* qpos, int32_t num_reqs,
                          int32_t max_tiles, void* out) {
  lazy_status st = check_geom(g);
  if (st != LAZY_OK) return st;
  st = check_pos(g, pd);
  if (st != LAZY_OK) return st;
  if (num_reqs < 0) return fail(LAZY_ERR_ARG, "num_reqs must be >= 0 (got %d)", num_reqs);
  if (max_tiles < 0) return fail(LAZY_ERR_ARG, "max_tiles must be >= 0 (got %d)", max_tiles);
  if (num_blocks < 1 || num_blocks > (int64_t)LAZY_MAX_BLOCK_ID + 1)
    return fail(LAZY_ERR_ARG, "num_blocks must be in [1, 2^24] (got %lld)", (long long)num_blocks);
  if (num_reqs > 0 && (!kc || !vc || !tiles || !tile_start || !ctx_tiles || !q || !qpos || !out))
    return fail(LAZY_ERR_ARG, "a required device pointer is NULL");
  if (num_reqs > 65535) return fail(LAZY_ERR_UNSUPPORTED, "num_reqs > 65535 is not supported");
  return LAZY_OK;
}

}  // namespace
}  // namespace lazy

using namespace lazy;

extern "C" size_t lazy_attn_workspace_size(const lazy_geom* geom, int32_t num_reqs, int32_t max_q_len,
                                           int32_t max_tiles, int32_t is_prefill) {
  if (check_geom(geom) != LAZY_OK || num_reqs <= 0 || max_tiles < 0) return 0;
  if (is_prefill && max_q_len <= 0) return 0;
  const Plan p = make_plan(geom, num_reqs, is_prefill ? max_q_len : 1, max_tiles, is_prefill != 0);
  return ws_bytes_for(geom, p);
}

extern "C" lazy_status lazy_attn_prefill(const lazy_geom* geom, const lazy_pos_desc* pos, const void* k_cache,
                                         const void* v_cache, int64_t num_blocks, const uint64_t* tiles,
                                         const int32_t* tile_start, const int32_t* ctx_tiles, const void* q,
                                         const int32_t* q_start, const int32_t* q_pos0, int32_t num_reqs,
                                         int32_t max_q_len, int32_t max_tiles, void* out, void* workspace,
                                         size_t ws_bytes, void* stream) {
  clear_error();
  lazy_status st = common_checks(geom, pos, k_cache, v_cache, num_blocks, tiles, tile_start, ctx_tiles, q, q_pos0,
                                 num_reqs, max_tiles, out);
  if (st != LAZY_OK) return st;
  if (num_reqs > 0 && !q_start) return fail(LAZY_ERR_ARG, "q_start is NULL");
  if (max_q_len < 0) return fail(LAZY_ERR_ARG, "max_q_len must be >= 0 (got %d)", max_q_len);
  if (num_reqs == 0 || max_q_len == 0) return LAZY_OK;
  const int group = geom->num_q_heads / geom->num_kv_heads;
  if ((int64_t)max_q_len * num_reqs * geom->num_q_heads > (int64_t)INT32_MAX / 2 ||
      (int64_t)max_q_len * group > (int64_t)INT32_MAX / 2)
    return fail(LAZY_ERR_UNSUPPORTED, "too many query rows");
  const Plan p = make_plan(geom, num_reqs, max_q_len, max_tiles, true);
  const size_t need = ws_bytes_for(geom, p);
  if (need > 0 && (workspace == nullptr || ws_bytes < need))
    return fail(LAZY_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  AttnArgs a{};
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_blocks = num_blocks;
  a.tiles = tiles;
  a.tile_start = tile_start;
  a.ctx_tiles = ctx_tiles;
  a.q = q;
  a.q_start = q_start;
  a.q_pos = q_pos0;
  a.cos_sin = pos->cos_sin;
  a.inv_freq = pos->inv_freq;
  a.max_pos = pos->max_pos;
  a.slopes = pos->alibi_slopes;
  a.scale_log2 = pos->softmax_scale * kLog2e;
  a.out = out;
  a.num_splits = p.splits;
  a.splits_per_wg = p.wt;
  a.hq = geom->num_q_heads;
  a.hkv = geom->num_kv_heads;
  a.group = group;
  a.rows_bound = p.rows_bound;
  a.max_q_len = max_q_len;
  if (need > 0) {
    a.part_o = reinterpret_cast<float*>(workspace);
    a.part_ml = a.part_o + (size_t)p.splits * p.rows_bound * geom->head_dim;
  }
  const hipError_t e = run<true>(geom, pos, a, p, num_reqs, q_start, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(LAZY_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
  return LAZY_OK;
}

extern "C" lazy_status lazy_attn_decode(const lazy_geom* geom, const lazy_pos_desc* pos, const void* k_cache,
                                        const void* v_cache, int64_t num_blocks, const uint64_t* tiles,
                                        const int32_t* tile_start, const int32_t* ctx_tiles, const void* q,
                                        const int32_t* q_pos, int32_t num_reqs, int32_t max_tiles, void* out,
                                        void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  lazy_status st = common_checks(geom, pos, k_cache, v_cache, num_blocks, tiles, tile_start, ctx_tiles, q, q_pos,
                                 num_reqs, max_tiles, out);
  if (st != LAZY_OK) return st;
  if (num_reqs == 0) return LAZY_OK;
  const Plan p = make_plan(geom, num_reqs, 1, max_tiles, false);
  const size_t need = ws_bytes_for(geom, p);
  if (need > 0 && (workspace == nullptr || ws_bytes < need))
    return fail(LAZY_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  AttnArgs a{};
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_blocks = num_blocks;
  a.tiles = tiles;
  a.tile_start = tile_start;
  a.ctx_tiles = ctx_tiles;
  a.q = q;
  a.q_start = nullptr;
  a.q_pos = q_pos;
  a.cos_sin = pos->cos_sin;
  a.inv_freq = pos->inv_freq;
  a.max_pos = pos->max_pos;
  a.slopes = pos->alibi_slopes;
  a.scale_log2 = pos->softmax_scale * kLog2e;
  a.out = out;
  a.num_splits = p.splits;
  a.splits_per_wg = p.wt;
  a.hq = geom->num_q_heads;
  a.hkv = geom->num_kv_heads;
  a.group = geom->num_q_heads / geom->num_kv_heads;
  a.rows_bound = p.rows_bound;
  a.max_q_len = 1;
  if (need > 0) {
    a.part_o = reinterpret_cast<float*>(workspace);
    a.part_ml = a.part_o + (size_t)p.splits * p.rows_bound * geom->head_dim;
  }
  const hipError_t e = run<false>(geom, pos, a, p, num_reqs, nullptr, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(LAZY_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return LAZY_OK;
}

extern "C" lazy_status lazy_debug_unpack(const uint64_t* words, int64_t n, int32_t* block, int32_t* offset,
                                         int32_t* mask, void* stream) {
  clear_error();
  if (n < 0) return fail(LAZY_ERR_ARG, "n must be >= 0");
  if (n == 0) return LAZY_OK;
  if (!words || !block || !offset || !mask) return fail(LAZY_ERR_ARG, "a device pointer is NULL");
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(debug_unpack_kernel, dim3(blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), words,
                     n, block, offset, mask);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(LAZY_ERR_HIP, "unpack launch failed: %s", hipGetErrorString(e));
  return LAZY_OK;
}
