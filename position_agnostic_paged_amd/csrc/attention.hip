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
#include <mutex>
#include <type_traits>

#include "attn_common.hpp"

namespace lazy {

// Prefill: one wave = RB blocks of 16 query rows x one split of the request's
// tiles; a workgroup = WR waves over consecutive row blocks (same split).
template <typename T, int DH, int KIND, bool DEFER, int RB, int WR>
__global__ __launch_bounds__(64 * WR) void prefill_kernel(AttnArgs a) {
  using W = WaveAttn<T, DH, KIND, DEFER, true, RB>;
  const int lane = threadIdx.x & 63;
#if LAZY_UNIFORM_WAVE
  const int wr = uniform(threadIdx.x >> 6);  // wave-uniform: keeps tile metadata in scalar registers
#else
  const int wr = threadIdx.x >> 6;
#endif
  const int req = blockIdx.z;
  const int kvh = blockIdx.y;
  const int row_tile = blockIdx.x / a.num_splits;
  const int split = blockIdx.x % a.num_splits;

  const int q0 = a.q_start[req];
  int nq = a.q_start[req + 1] - q0;
  // never address query rows beyond what the grid and workspace were sized for
  nq = min(nq, a.max_q_len);
  nq = max(0, min(nq, a.rows_bound / a.hq - q0));
  const int nrows = nq * a.group;
  const int rb0 = (row_tile * WR + wr) * RB;
  if (rb0 * 16 >= nrows) return;  // no rows for this wave (no barriers follow)

  const int nt = a.tile_start[req + 1] - a.tile_start[req];
  int sb, se;
  if (!split_range(nt, a.chunk, a.num_splits, split, sb, se)) return;  // unused split (no barriers follow)
  W w(a, lane, kvh, req, q0, nrows, rb0, a.q_pos[req]);
  const int npairs = (se - sb + 1) >> 1;
  for (int p = 0; p < npairs; ++p) {
    const typename W::Pair pr = w.read_pair(sb + 2 * p, se);
    typename W::Frags f;
    w.load(pr, f);
    w.rotate_for(pr);
    w.consume(pr, f);
  }
  w.finalize(split);
}

// Decode: one wave = the G query heads of one (request, KV head) x one split;
// a workgroup = WT waves on WT consecutive splits.  Each tile pair's K/V is
// loaded, then consumed, with the next pair's tile words fetched one pair
// ahead; LAZY_DECODE_PIPELINE builds the variant that keeps the next pair's
// K/V loads in flight during the products instead (more registers per wave,
// so fewer waves: slower on this part).
// Grid (KV head, request, split group), fastest first.  Dispatch deals
// consecutive workgroups round-robin over the 8 XCDs, so with 8 KV heads
// every XCD (its own L2) serves one head, and all requests that read a shared
// document's block read that head's slice through the same L2.  Split groups
// are the slowest dimension, so the first splits of every request run
// together: with the host listing each request's documents most shared
// first, a shared document is read for all its requests at about the same
// time and mostly comes from L2 after the first read.
// WPE > 1 asks the compiler for at least WPE resident waves per SIMD (a
// register cap): the launch picks it for uneven batches, whose many short
// splits gain from more waves in flight.
template <typename T, int DH, int KIND, bool DEFER, int RB, int WT, int WPE>
__global__ __launch_bounds__(64 * WT) __attribute__((amdgpu_waves_per_eu(WPE))) void decode_kernel(AttnArgs a) {
  using W = WaveAttn<T, DH, KIND, DEFER, false, RB>;
  const int lane = threadIdx.x & 63;
#if LAZY_UNIFORM_WAVE
  const int wt = uniform(threadIdx.x >> 6);  // wave-uniform: keeps tile metadata in scalar registers
#else
  const int wt = threadIdx.x >> 6;
#endif
  const int req = blockIdx.y;
  const int kvh = blockIdx.x;
  const int split = blockIdx.z * WT + wt;
  const int nt = a.tile_start[req + 1] - a.tile_start[req];
  int sb, se;
  if (!split_range(nt, a.chunk, a.num_splits, split, sb, se)) return;  // unused split (no barriers follow)

  W w(a, lane, kvh, req, req, a.group, 0, a.q_pos[req]);
  const int npairs = (se - sb + 1) >> 1;
#if LAZY_DECODE_PIPELINE
  if (npairs > 0) {
    typename W::Pair pa = w.read_pair(sb, se), pb;
    typename W::Frags fa, fb;
    w.load(pa, fa);
    for (int p = 0;; p += 2) {
      const bool more = p + 1 < npairs;
      if (more) {
        pb = w.read_pair(sb + 2 * (p + 1), se);
        w.load(pb, fb);
      }
      w.rotate_for(pa);
      w.consume(pa, fa);
      if (!more) break;
      const bool more2 = p + 2 < npairs;
      if (more2) {
        pa = w.read_pair(sb + 2 * (p + 2), se);
        w.load(pa, fa);
      }
      w.rotate_for(pb);
      w.consume(pb, fb);
      if (!more2) break;
    }
  }
#else
  // the next pair's tile words are fetched one iteration ahead
  uint64_t w0 = 0, w1 = 0;
  if (npairs > 0) w.fetch_words(sb, se, w0, w1);
  for (int p = 0; p < npairs; ++p) {
    const typename W::Pair pr = w.decode_pair(sb + 2 * p, se, w0, w1);
    if (p + 1 < npairs) w.fetch_words(sb + 2 * (p + 1), se, w0, w1);
    w.rotate_for(pr);
    typename W::Frags f;
    w.load(pr, f);
    w.consume(pr, f);
  }
#endif
  w.finalize(split);
}

// Document-major decode pass: one wave = RB blocks of 16 rows of one shared
// document for one KV head, a row being one request's read of the document
// (at that request's offset Delta) x one query head of the group.  The
// document's tiles are read once for all those rows; each row's query is
// rotated once, by -Delta of its read, and the keys stay at their local
// positions (the single relative rotation, applied per reader).  A long
// document is cut into chunks of tiles, one wave each, so a few documents
// with many readers still fill the chip.  Every row ends as an (m, l, acc)
// partial in its request's slot (one per chunk), merged with the request's
// other partials by the combine.  Grid (KV head, work item): one
// head per XCD, and a document's row blocks are adjacent work items, so the
// waves reading one document's head slice share an L2.
template <typename T, int DH, int KIND, int RB, int WPE>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(WPE))) void docpass_kernel(AttnArgs a,
                                                                                               DocPassArgs d) {
  using W = WaveAttn<T, DH, KIND, false, false, RB>;
  const int lane = threadIdx.x & 63;
  const int kvh = blockIdx.x;
  const int item = blockIdx.y;
  const int doc = d.work[4 * item];
  const int rb0 = d.work[4 * item + 1];
  const int chunk = d.work[4 * item + 2];
  const int chunk_tiles = d.work[4 * item + 3];
  const int nrows = (d.read_start[doc + 1] - d.read_start[doc]) * a.group;
  if (rb0 * 16 >= nrows || chunk_tiles < 1) return;
  W w(a, d, lane, kvh, doc, nrows, rb0, chunk, chunk_tiles, typename W::DocRows{});
  const int nt = w.nctx;
  const int npairs = (nt + 1) >> 1;
  uint64_t w0 = 0, w1 = 0;
  if (npairs > 0) w.fetch_words(0, nt, w0, w1);
  for (int p = 0; p < npairs; ++p) {
    const typename W::Pair pr = w.decode_pair(2 * p, nt, w0, w1);
    if (p + 1 < npairs) w.fetch_words(2 * (p + 1), nt, w0, w1);
    typename W::Frags f;
    w.load(pr, f);
    w.consume(pr, f);
  }
  w.finalize(0);
}

// Split-K combine (flash-decoding): for every output row,
//   M = max_s m_s,  out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s,
// over the splits its request used.  Splits that saw no visible key carry
// m = -inf and contribute nothing.
template <typename T, int DH, int NG>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml, T* __restrict__ out,
                                                      const int32_t* __restrict__ q_start,
                                                      const int32_t* __restrict__ tile_start, int32_t num_reqs,
                                                      int32_t hq, int32_t rows_bound, int32_t max_splits,
                                                      int32_t chunk, const int32_t* __restrict__ extra_n,
                                                      int32_t extra_base, const bf16* __restrict__ extra_o) {
  // RPB rows per workgroup; per row, TPR threads cover the channels (4 each)
  // and NG groups of them take every NG-th split, so the partial loads of
  // many splits are in flight together (NG = 1 for few splits); the groups'
  // maxima, weighted sums and vectors meet in LDS.
  constexpr int TPR = DH / 4;
  constexpr int RPB = 256 / (TPR * NG);
  static_assert(RPB >= 1 && RPB * TPR * NG == 256, "combine shape");
  __shared__ float red_m[RPB][NG], red_l[RPB][NG];
  __shared__ f32x4 red_o[RPB][NG][TPR];
  const int rr = threadIdx.x / (TPR * NG);
  const int row = blockIdx.x * RPB + rr;
  const int grp = (threadIdx.x / TPR) % NG;
  const int ct = threadIdx.x % TPR;
  const int c4 = ct * 4;
  const int rows = min(rows_bound, (q_start != nullptr) ? q_start[num_reqs] * hq : num_reqs * hq);
  if (row >= rows) return;  // uniform over the row's threads; barriers below only when NG > 1 (RPB = 1)
  int req;
  const int qrow = row / hq;
  if (q_start == nullptr) {
    req = qrow;  // decode: one query row per request
  } else {       // prefill: the request whose row range holds qrow
    int lo = 0, hi = num_reqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (q_start[mid] <= qrow) lo = mid; else hi = mid - 1;
    }
    req = lo;
  }
  // max_splits 0: no split partials (a document-major decode with no own tiles)
  const int ns = max_splits > 0 ? request_splits(tile_start[req + 1] - tile_start[req], chunk, max_splits) : 0;
  // One pass: each group merges its splits into a running (m, l, o),
  // rescaling when the maximum grows, so every partial load is independent
  // of the others (an empty split, m = -inf, has weight 0).
  float M = -INFINITY, L = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  // the request's split partials, then (document-major decode) its partials
  // from the shared-document pass in slots extra_base ..
  const int ne = (extra_n != nullptr) ? extra_n[req] : 0;
  for (int s = grp; s < ns + ne; s += NG) {
    const int64_t pr = (int64_t)(s < ns ? s : extra_base + (s - ns)) * rows_bound + row;
    const float ms = part_ml[pr * 2], ls = part_ml[pr * 2 + 1];
    f32x4 os;
    if (extra_o != nullptr && s >= ns) {  // a bf16 accumulator of the document pass
      const bf16x4 e = *reinterpret_cast<const bf16x4*>(extra_o + ((int64_t)(s - ns) * rows_bound + row) * DH + c4);
#pragma unroll
      for (int j = 0; j < 4; ++j) os[j] = (float)e[j];
    } else {
      os = *reinterpret_cast<const f32x4*>(part_o + pr * DH + c4);
    }
    const float mn = fmaxf(M, ms);
    const float a = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - mn);
    const float b = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - mn);
    o = o * a + os * b;
    L = L * a + ls * b;
    M = mn;
  }
  if constexpr (NG > 1) {
    if (ct == 0) {
      red_m[rr][grp] = M;
      red_l[rr][grp] = L;
    }
    red_o[rr][grp][ct] = o;
    __syncthreads();
    if (grp != 0) return;
    float Mt = red_m[rr][0];
#pragma unroll
    for (int i = 1; i < NG; ++i) Mt = fmaxf(Mt, red_m[rr][i]);
    o = f32x4{0.f, 0.f, 0.f, 0.f};
    L = 0.f;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const float mi = red_m[rr][i];
      const float w = (mi == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mi - Mt);
      o += w * red_o[rr][i][ct];
      L += w * red_l[rr][i];
    }
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

constexpr int kPrefillWR = 4;  // waves per prefill workgroup (each RB x 16 query rows)
// one wave (one split) per workgroup: on the uneven mixed batch 791 us vs 798
// (two) / 812 (four) / 862 (eight); near-uniform no-sharing batch unchanged
constexpr int kDecodeWT = 1;

// 16-row blocks per decode wave: the smallest count that holds the G query
// heads of a KV head (Falcon's MQA 71 heads: 5 blocks, 80 rows, instead of
// 128 rows of which 57 would be padding)
int decode_rb(int group) {
#if LAZY_DECODE_RB_EXACT
  return group <= 16 ? 1 : group <= 32 ? 2 : group <= 48 ? 3 : group <= 64 ? 4 : group <= 80 ? 5 : 8;
#else
  return group <= 16 ? 1 : group <= 32 ? 2 : group <= 64 ? 4 : 8;
#endif
}

struct Plan {
  int rb, wr, wt;
  bool uneven;  // decode: request lengths far apart (more, shorter splits)
  int row_tiles;
  int splits;  // grid extent along splits
  int chunk;   // tiles per split
  int rows_bound;
};

// Tiles per split so that about `target` work items (waves for decode,
// workgroups for prefill) cover total_tiles x (KV heads x row tiles); each
// request then uses ceil(its tiles / chunk) splits, which balances requests of
// very different lengths.  total_tiles <= 0 means "unknown" (num_reqs x max_tiles).
void size_splits(Plan& p, long per_tile_units, int num_reqs, int max_tiles, int64_t total_tiles, long target,
                 int min_chunk) {
  const long T = total_tiles > 0 ? (long)total_tiles : (long)num_reqs * max_tiles;
  long chunk = (T * per_tile_units + target - 1) / std::max(1L, target);
  chunk = std::max<long>(chunk, min_chunk);
  const int max_splits = 256;
  if ((max_tiles + chunk - 1) / chunk > max_splits) chunk = (max_tiles + max_splits - 1) / max_splits;
  chunk = (chunk + 1) & ~1L;  // whole tile pairs
  p.chunk = (int)std::min<long>(chunk, 1 << 30);
  p.splits = std::max(1, (int)((max_tiles + p.chunk - 1) / p.chunk));
}

Plan make_plan(const lazy_geom* g, int num_reqs, int max_q_len, int max_tiles, int64_t total_tiles, bool prefill) {
  Plan p;
  p.uneven = false;
  const int group = g->num_q_heads / g->num_kv_heads;
  if (prefill) {
    // 4 row blocks per wave when a request has >= 256 query rows (halves the
    // LDS bytes per MFMA of the staged kernel), else 2
    p.rb = (max_q_len * group >= 256) ? 4 : 2;
    p.wr = kPrefillWR;
    p.wt = 1;
    const int rows = max_q_len * group;
    p.row_tiles = (rows + 16 * p.rb * p.wr - 1) / (16 * p.rb * p.wr);
    size_splits(p, (long)g->num_kv_heads * p.row_tiles, num_reqs, max_tiles, total_tiles, LAZY_PREFILL_WG_TARGET, 16);
    p.rows_bound = max_q_len * num_reqs * g->num_q_heads;
  } else {
    p.rb = decode_rb(group);
    p.wr = 1;
    p.wt = kDecodeWT;
    p.row_tiles = 1;
    p.uneven = total_tiles > 0 && (double)max_tiles * num_reqs > 1.25 * (double)total_tiles;
    size_splits(p, g->num_kv_heads, num_reqs, max_tiles, total_tiles,
                p.uneven ? LAZY_DECODE_WAVE_TARGET_UNEVEN : LAZY_DECODE_WAVE_TARGET, LAZY_DECODE_MIN_CHUNK);
    p.rows_bound = num_reqs * g->num_q_heads;
  }
  return p;
}

size_t ws_bytes_for(const lazy_geom* g, const Plan& p) {
  if (p.splits == 1) return 0;
  const size_t per = (size_t)g->head_dim + 2;
  return (size_t)p.splits * (size_t)p.rows_bound * per * sizeof(float) + 256;
}

// Largest split count whose partials fit `cap` bytes (0 if not even two do).
int splits_within(const lazy_geom* g, const Plan& p, size_t cap) {
  const size_t per_split = (size_t)p.rows_bound * ((size_t)g->head_dim + 2) * sizeof(float);
  if (cap < 256 + 2 * per_split) return 0;
  return (int)std::min<size_t>((cap - 256) / per_split, 1 << 20);
}

// The same plan with fewer, longer splits so that its partials fit `cap`
// bytes (fewer splits only lengthen each wave's tile range).
void cap_splits(Plan& p, int max_splits, int max_tiles) {
  if (p.splits <= max_splits) return;
  long chunk = ((long)max_tiles + max_splits - 1) / max_splits;
  chunk = (chunk + 1) & ~1L;  // whole tile pairs
  p.chunk = (int)chunk;
  p.splits = std::max(1, (int)((max_tiles + chunk - 1) / chunk));
}

template <typename T, int DH, int KIND, bool DEFER, int RB>
hipError_t launch_decode(const AttnArgs& a, const Plan& p, int num_reqs, int hkv, hipStream_t st) {
  dim3 grid((unsigned)hkv, (unsigned)num_reqs, (unsigned)((p.splits + kDecodeWT - 1) / kDecodeWT));
  // bf16 with one row block fits three waves per SIMD without spilling (168
  // VGPRs, 200 uncapped); uneven batches run that build, near-uniform ones,
  // which one resident round of two waves per SIMD serves best, the other
  if constexpr (std::is_same<T, bf16>::value && RB == 1) {
    if (p.uneven) {
      hipLaunchKernelGGL((decode_kernel<T, DH, KIND, DEFER, RB, kDecodeWT, 3>), grid, dim3(64 * kDecodeWT), 0, st, a);
      return hipGetLastError();
    }
  }
  // several row blocks of dh 64 (large query groups, MQA): capped at two
  // waves per SIMD, which the uncapped build's 300+ registers would not
  // allow (at dh 128 the cap spills hundreds of registers: not used)
  if constexpr (RB >= 3 && DH == 64 && LAZY_DECODE_MANY_ROWS_WPE > 1) {
    hipLaunchKernelGGL((decode_kernel<T, DH, KIND, DEFER, RB, kDecodeWT, LAZY_DECODE_MANY_ROWS_WPE>), grid,
                       dim3(64 * kDecodeWT), 0, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((decode_kernel<T, DH, KIND, DEFER, RB, kDecodeWT, 1>), grid, dim3(64 * kDecodeWT), 0, st, a);
  return hipGetLastError();
}

template <typename T, int DH, int KIND, bool DEFER, bool PREFILL>
hipError_t dispatch_rb(const AttnArgs& a, const Plan& p, int num_reqs, int hkv, hipStream_t st) {
  if (PREFILL) {
    // bf16 with a cos/sin table (or no rotation): the LDS-staged kernel
    if (std::is_same<T, bf16>::value) {
      const hipError_t e = launch_prefill_lds(a, KIND, DEFER, DH, p.rb, p.row_tiles, p.splits, num_reqs, hkv, st);
      if (e != hipErrorNotSupported) return e;
    }
    dim3 grid((unsigned)(p.row_tiles * p.splits), (unsigned)hkv, (unsigned)num_reqs);
    if (p.rb == 4)
      hipLaunchKernelGGL((prefill_kernel<T, DH, KIND, DEFER, 4, kPrefillWR>), grid, dim3(64 * kPrefillWR), 0, st, a);
    else
      hipLaunchKernelGGL((prefill_kernel<T, DH, KIND, DEFER, 2, kPrefillWR>), grid, dim3(64 * kPrefillWR), 0, st, a);
    return hipGetLastError();
  }
  switch (p.rb) {
    case 1:
      return launch_decode<T, DH, KIND, DEFER, 1>(a, p, num_reqs, hkv, st);
    case 2:
      return launch_decode<T, DH, KIND, DEFER, 2>(a, p, num_reqs, hkv, st);
    case 3:
      return launch_decode<T, DH, KIND, DEFER, 3>(a, p, num_reqs, hkv, st);
    case 4:
      return launch_decode<T, DH, KIND, DEFER, 4>(a, p, num_reqs, hkv, st);
    case 5:
      return launch_decode<T, DH, KIND, DEFER, 5>(a, p, num_reqs, hkv, st);
    default:
      return launch_decode<T, DH, KIND, DEFER, 8>(a, p, num_reqs, hkv, st);
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
hipError_t launch_combine(const AttnArgs& a, const Plan& p, const int32_t* q_start, int num_reqs, hipStream_t st,
                          const int32_t* extra_n = nullptr, int extra_base = 0, int max_extra = 0,
                          const bf16* extra_o = nullptr) {
  // many partials per row: one row per workgroup, 256 / (DH/4) split groups;
  // few: rows side by side
  constexpr int NGMAX = 256 / (DH / 4);
  if (p.splits + max_extra > 4) {
    dim3 grid((unsigned)p.rows_bound);
    hipLaunchKernelGGL((combine_kernel<T, DH, NGMAX>), grid, dim3(256), 0, st, a.part_o, a.part_ml,
                       reinterpret_cast<T*>(a.out), q_start, a.tile_start, num_reqs, a.hq, p.rows_bound, p.splits,
                       p.chunk, extra_n, extra_base, extra_o);
  } else {
    constexpr int RPB = NGMAX;
    dim3 grid((unsigned)((p.rows_bound + RPB - 1) / RPB));
    hipLaunchKernelGGL((combine_kernel<T, DH, 1>), grid, dim3(256), 0, st, a.part_o, a.part_ml,
                       reinterpret_cast<T*>(a.out), q_start, a.tile_start, num_reqs, a.hq, p.rows_bound, p.splits,
                       p.chunk, extra_n, extra_base, extra_o);
  }
  return hipGetLastError();
}

// The document pass for one (dtype, head_dim, kind).
template <typename T, int DH, int KIND>
hipError_t launch_docpass(const AttnArgs& a, const DocPassArgs& d, int rb, int num_work, int hkv, hipStream_t st) {
  dim3 grid((unsigned)hkv, (unsigned)num_work);
  // the row blocks docpass_row_blocks gives: 2 at dh 128, 4 at dh 64 (both
  // within two waves per SIMD)
  constexpr int RB = (DH == 128) ? LAZY_DOCPASS_RB128 : 4;
  if (rb != RB) return hipErrorNotSupported;
  hipLaunchKernelGGL((docpass_kernel<T, DH, KIND, RB, LAZY_DOCPASS_WPE>), grid, dim3(64), 0, st, a, d);
  return hipGetLastError();
}

template <typename T, int DH>
hipError_t docpass_kind(int kind, const AttnArgs& a, const DocPassArgs& d, int rb, int num_work, int hkv,
                        hipStream_t st) {
  switch (kind) {
    case kHalf:
      return launch_docpass<T, DH, kHalf>(a, d, rb, num_work, hkv, st);
    case kInter:
      return launch_docpass<T, DH, kInter>(a, d, rb, num_work, hkv, st);
    default:
      return launch_docpass<T, DH, kAlibi>(a, d, rb, num_work, hkv, st);
  }
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
  const int32_t* qs = PREFILL ? q_start : nullptr;
  if (g->dtype == LAZY_BF16)
    return (g->head_dim == 128) ? launch_combine<bf16, 128>(a, p, qs, num_reqs, st)
                                : launch_combine<bf16, 64>(a, p, qs, num_reqs, st);
  return (g->head_dim == 128) ? launch_combine<float, 128>(a, p, qs, num_reqs, st)
                              : launch_combine<float, 64>(a, p, qs, num_reqs, st);
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
                                           int32_t max_tiles, int64_t total_tiles, int32_t is_prefill) {
  if (check_geom(geom) != LAZY_OK || num_reqs <= 0 || max_tiles < 0) return 0;
  if (is_prefill && max_q_len <= 0) return 0;
  const Plan p = make_plan(geom, num_reqs, is_prefill ? max_q_len : 1, max_tiles, total_tiles, is_prefill != 0);
  return ws_bytes_for(geom, p);
}

extern "C" lazy_status lazy_attn_prefill(const lazy_geom* geom, const lazy_pos_desc* pos, const void* k_cache,
                                         const void* v_cache, int64_t num_blocks, const uint64_t* tiles,
                                         const int32_t* tile_start, const int32_t* ctx_tiles, const void* q,
                                         const int32_t* q_start, const int32_t* q_pos0, int32_t num_reqs,
                                         int32_t max_q_len, int32_t max_tiles, int64_t total_tiles, void* out,
                                         void* workspace,
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
  const Plan p = make_plan(geom, num_reqs, max_q_len, max_tiles, total_tiles, true);
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
  a.chunk = p.chunk;
  a.hq = geom->num_q_heads;
  a.hkv = geom->num_kv_heads;
  a.group = group;
  a.rows_bound = p.rows_bound;
  a.max_q_len = max_q_len;
  a.doc_pairs = (pos->flags & LAZY_FLAG_DOC_PAIRS) ? 1 : 0;
  if (need > 0) {
    a.part_o = reinterpret_cast<float*>(workspace);
    a.part_ml = a.part_o + (size_t)p.splits * p.rows_bound * geom->head_dim;
  }
  const hipError_t e = run<true>(geom, pos, a, p, num_reqs, q_start, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(LAZY_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
  return LAZY_OK;
}

namespace lazy {
namespace {

// The decode plan; with scratch_cap > 0 its partials must fit that many
// bytes (fewer, longer splits when the default plan needs more; refused when
// not even two splits fit).  Host only.
lazy_status plan_decode(const lazy_geom* geom, int32_t num_reqs, int32_t max_tiles, int64_t total_tiles,
                        size_t scratch_cap, Plan& p) {
  p = make_plan(geom, num_reqs, 1, max_tiles, total_tiles, false);
  if (scratch_cap > 0 && ws_bytes_for(geom, p) > scratch_cap) {
    const int fit = splits_within(geom, p, scratch_cap);
    if (fit < 2)
      return fail(LAZY_ERR_WORKSPACE,
                  "%d query rows need %zu bytes for two splits' partials; the static scratch holds %zu",
                  p.rows_bound, 2 * (size_t)p.rows_bound * ((size_t)geom->head_dim + 2) * sizeof(float) + 256,
                  scratch_cap);
    cap_splits(p, fit, max_tiles);
  }
  return LAZY_OK;
}

// Decode with a caller-given workspace (scratch_cap == 0) or with the
// library's static scratch (scratch_cap = its size: the plan is capped to fit).
lazy_status decode_impl(const lazy_geom* geom, const lazy_pos_desc* pos, const void* k_cache, const void* v_cache,
                        int64_t num_blocks, const uint64_t* tiles, const int32_t* tile_start,
                        const int32_t* ctx_tiles, const void* q, const int32_t* q_pos, int32_t num_reqs,
                        int32_t max_tiles, int64_t total_tiles, void* out, void* workspace, size_t ws_bytes,
                        size_t scratch_cap, void* stream) {
  lazy_status st = common_checks(geom, pos, k_cache, v_cache, num_blocks, tiles, tile_start, ctx_tiles, q, q_pos,
                                 num_reqs, max_tiles, out);
  if (st != LAZY_OK) return st;
  if (num_reqs == 0) return LAZY_OK;
  Plan p;
  st = plan_decode(geom, num_reqs, max_tiles, total_tiles, scratch_cap, p);
  if (st != LAZY_OK) return st;
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
  a.chunk = p.chunk;
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

// ------------------------------------------------ static scratch (no-allocation decode)
//
// The split-K partials of lazy_attn_decode_noalloc live in this file-scope
// device array: every GPU the library runs on holds its own copy for the
// life of the process.  Host code never passes the array's name to a kernel
// (on the host it is only a stand-in symbol): its device address is looked
// up once per device, with that device current, and kept here.
static __device__ __align__(256) unsigned char scratch[LAZY_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

lazy_status scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(LAZY_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(LAZY_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(LAZY_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LAZY_OK;
}

}  // namespace
}  // namespace lazy

extern "C" lazy_status lazy_attn_decode(const lazy_geom* geom, const lazy_pos_desc* pos, const void* k_cache,
                                        const void* v_cache, int64_t num_blocks, const uint64_t* tiles,
                                        const int32_t* tile_start, const int32_t* ctx_tiles, const void* q,
                                        const int32_t* q_pos, int32_t num_reqs, int32_t max_tiles,
                                        int64_t total_tiles, void* out,
                                        void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  return decode_impl(geom, pos, k_cache, v_cache, num_blocks, tiles, tile_start, ctx_tiles, q, q_pos, num_reqs,
                     max_tiles, total_tiles, out, workspace, ws_bytes, 0, stream);
}

extern "C" lazy_status lazy_attn_decode_noalloc(const lazy_geom* geom, const lazy_pos_desc* pos, const void* k_cache,
                                                const void* v_cache, int64_t num_blocks, const uint64_t* tiles,
                                                const int32_t* tile_start, const int32_t* ctx_tiles, const void* q,
                                                const int32_t* q_pos, int32_t num_reqs, int32_t max_tiles,
                                                int64_t total_tiles, void* out, void* stream) {
  clear_error();
  // arguments first: nothing touches the device for a call that would be refused
  lazy_status st = common_checks(geom, pos, k_cache, v_cache, num_blocks, tiles, tile_start, ctx_tiles, q, q_pos,
                                 num_reqs, max_tiles, out);
  if (st != LAZY_OK || num_reqs == 0) return st;
  Plan p;
  st = plan_decode(geom, num_reqs, max_tiles, total_tiles, LAZY_NOALLOC_SCRATCH_BYTES, p);  // refusals first
  if (st != LAZY_OK) return st;
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != LAZY_OK) return st;
  return decode_impl(geom, pos, k_cache, v_cache, num_blocks, tiles, tile_start, ctx_tiles, q, q_pos, num_reqs,
                     max_tiles, total_tiles, out, ws, LAZY_NOALLOC_SCRATCH_BYTES, LAZY_NOALLOC_SCRATCH_BYTES, stream);
}

namespace lazy {
namespace {

// Workspace of the document-major decode: (m, l) of every partial slot in
// fp32; the split slots' accumulators in fp32; the document pass's slots'
// accumulators in the call's dtype (bf16 halves the pass's partial traffic,
// written once and read once by the combine, for a rounding like the
// output's own).
size_t shared_ws_doc_bytes(const lazy_geom* g, const Plan& p, int max_req_reads) {
  const size_t esz = g->dtype == LAZY_BF16 ? 2 : 4;
  return (size_t)max_req_reads * (size_t)p.rows_bound * (size_t)g->head_dim * esz;
}

size_t shared_ws_bytes(const lazy_geom* g, const Plan& p, int max_req_reads) {
  const size_t split_o = (size_t)p.splits * (size_t)p.rows_bound * (size_t)g->head_dim * sizeof(float);
  const size_t ml = (size_t)(p.splits + max_req_reads) * (size_t)p.rows_bound * 2 * sizeof(float);
  return split_o + ((shared_ws_doc_bytes(g, p, max_req_reads) + 255) & ~(size_t)255) + ml + 512;
}

template <typename T, int DH>
hipError_t run_shared(const lazy_pos_desc* pd, const AttnArgs& a, const DocPassArgs& d, const Plan& p, int rb,
                      int num_work, int num_reqs, int hkv, const int32_t* req_reads, int max_req_reads,
                      int64_t total_tiles, hipStream_t st) {
  // 1. each request's own tiles (unshared documents, private tokens), split-K
  //    as usual, always into partials; none when every one of them went to
  //    the pass (a plan with min_readers 1): no launch, and the combine
  //    reads no split partials
  Plan pc = p;
  hipError_t e = hipSuccess;
  if (total_tiles > 0) {
    e = dispatch_kind<T, DH, false>(pd->kind, true, a, p, num_reqs, hkv, st);
    if (e != hipSuccess) return e;
  } else {
    pc.splits = 0;
  }
  // 2. every shared document once for all its readers
  if (num_work > 0) {
    AttnArgs ad = a;
    ad.tiles = d.doc_tiles;
    ad.tile_start = d.doc_tile_start;
    if constexpr (std::is_same<T, bf16>::value && LAZY_DOCPASS_LDS)
      e = launch_docpass_lds(ad, d, pd->kind, DH, num_work, hkv, st);
    else
      e = docpass_kind<T, DH>(pd->kind, ad, d, rb, num_work, hkv, st);
    if (e != hipSuccess) return e;
  }
  // 3. per (request, head): the request's split partials and its reads' partials
  const bf16* doc_o = nullptr;
  if constexpr (std::is_same<T, bf16>::value) doc_o = reinterpret_cast<const bf16*>(d.doc_o);
  return launch_combine<T, DH>(a, pc, nullptr, num_reqs, st, req_reads, d.slot_base, max_req_reads, doc_o);
}

}  // namespace
}  // namespace lazy

extern "C" size_t lazy_attn_decode_shared_workspace_size(const lazy_geom* geom, int32_t num_reqs, int32_t max_tiles,
                                                        int64_t total_tiles, int32_t max_req_reads) {
  if (check_geom(geom) != LAZY_OK || num_reqs <= 0 || max_tiles < 0 || max_req_reads < 0) return 0;
  const Plan p = make_plan(geom, num_reqs, 1, max_tiles, total_tiles, false);
  return shared_ws_bytes(geom, p, max_req_reads);
}

extern "C" lazy_status lazy_attn_decode_shared(
    const lazy_geom* geom, const lazy_pos_desc* pos, const void* k_cache, const void* v_cache, int64_t num_blocks,
    const uint64_t* tiles, const int32_t* tile_start, const int32_t* ctx_tiles, int32_t max_tiles, int64_t total_tiles,
    const uint64_t* doc_tiles, const int32_t* doc_tile_start, const int32_t* read_start, const uint64_t* reads,
    const int32_t* req_reads, const int32_t* work, int32_t num_docs, int32_t num_work, int32_t max_req_reads,
    int32_t row_blocks, const void* q, const int32_t* q_pos, int32_t num_reqs, void* out, void* workspace,
    size_t ws_bytes, void* stream) {
  clear_error();
  lazy_status st = common_checks(geom, pos, k_cache, v_cache, num_blocks, tiles, tile_start, ctx_tiles, q, q_pos,
                                 num_reqs, max_tiles, out);
  if (st != LAZY_OK) return st;
  if (pos->flags & LAZY_FLAG_PREROTATED)
    return fail(LAZY_ERR_ARG, "the shared-document decode needs position-agnostic documents (no pre-rotated flag)");
  if (num_docs < 0 || num_work < 0 || max_req_reads < 0 || max_req_reads > 65536)
    return fail(LAZY_ERR_ARG, "num_docs, num_work >= 0 and max_req_reads in [0, 65536] required");
  if (row_blocks != docpass_row_blocks(geom))
    return fail(LAZY_ERR_ARG, "the plan was built for %d row blocks per work item; this geometry runs %d", row_blocks,
                docpass_row_blocks(geom));
  if (num_work > 65535) return fail(LAZY_ERR_UNSUPPORTED, "too many document work items (%d > 65535)", num_work);
  if (num_work > 0 && (!doc_tiles || !doc_tile_start || !read_start || !reads || !work))
    return fail(LAZY_ERR_ARG, "a document-pass array is NULL");
  if (num_reqs > 0 && !req_reads) return fail(LAZY_ERR_ARG, "req_reads is NULL");
  if (num_reqs == 0) return LAZY_OK;
  const Plan p = make_plan(geom, num_reqs, 1, max_tiles, total_tiles, false);
  const size_t need = shared_ws_bytes(geom, p, max_req_reads);
  if (workspace == nullptr || ws_bytes < need)
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
  a.chunk = p.chunk;
  a.hq = geom->num_q_heads;
  a.hkv = geom->num_kv_heads;
  a.group = geom->num_q_heads / geom->num_kv_heads;
  a.rows_bound = p.rows_bound;
  a.max_q_len = 1;
  a.force_partials = 1;
  // workspace: split accumulators (fp32) | document-pass accumulators (dtype)
  // | (m, l) of every slot; the document pass's slots are split slots
  // slot_base.. in part_ml and doc_o's own rows (fp32: they continue part_o)
  unsigned char* wsb = reinterpret_cast<unsigned char*>(workspace);
  const size_t split_o = (size_t)p.splits * p.rows_bound * geom->head_dim * sizeof(float);
  const size_t doc_bytes = (shared_ws_doc_bytes(geom, p, max_req_reads) + 255) & ~(size_t)255;
  a.part_o = reinterpret_cast<float*>(wsb);
  a.part_ml = reinterpret_cast<float*>(wsb + split_o + doc_bytes);
  DocPassArgs d{};
  d.doc_o = wsb + split_o;
  d.doc_tiles = doc_tiles;
  d.doc_tile_start = doc_tile_start;
  d.read_start = read_start;
  d.reads = reads;
  d.work = work;
  d.slot_base = p.splits;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int rb = row_blocks, hkv = geom->num_kv_heads;
  hipError_t e;
  if (geom->dtype == LAZY_BF16)
    e = geom->head_dim == 128
            ? run_shared<bf16, 128>(pos, a, d, p, rb, num_work, num_reqs, hkv, req_reads, max_req_reads, total_tiles, s)
            : run_shared<bf16, 64>(pos, a, d, p, rb, num_work, num_reqs, hkv, req_reads, max_req_reads, total_tiles, s);
  else
    e = geom->head_dim == 128
            ? run_shared<float, 128>(pos, a, d, p, rb, num_work, num_reqs, hkv, req_reads, max_req_reads, total_tiles, s)
            : run_shared<float, 64>(pos, a, d, p, rb, num_work, num_reqs, hkv, req_reads, max_req_reads, total_tiles, s);
  if (e != hipSuccess) return fail(LAZY_ERR_HIP, "shared-document decode launch failed: %s", hipGetErrorString(e));
  (void)num_docs;
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
