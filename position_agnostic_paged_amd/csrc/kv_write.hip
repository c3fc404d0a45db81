// KV-write path: position-agnostic document keys, private keys/queries at
// global positions (LazyAttention notes, papernotes.org, "Method: overall
// framework": each cached document is indexed from local position 0; the
// deferred offset is applied later inside attention.  The question and
// generated tokens keep ordinary RoPE at their global positions).
//
// One thread owns 8 rotation pairs (16 channels) of one (token, head) row:
//   K : cache slot <- R_pos k   (ALiBi: plain copy)
//   V : cache slot <- v         (channel-major block layout [dh][16])
//   Q : q          <- R_pos q   in place (optional)
// Coefficients come from one cos/sin table row per token (or fp64 sincos
// when no table is given).  Rotation in fp32; one rounding to the storage type.
#include <math.h>

#include <algorithm>

#include "lazy_device.hpp"
#include "lazy_host.hpp"

namespace lazy {

struct KvArgs {
  void* k_cache;
  void* v_cache;
  int64_t num_slots;  // num_blocks * 16
  const void* k;
  const void* v;
  void* q;
  const int32_t* positions;
  const int64_t* slots;
  const float* cos_sin;
  const double* inv_freq;
  int32_t max_pos;
  int32_t num_tokens;
  int32_t hq, hkv;
};

enum { kvHalf = LAZY_ROPE_HALF, kvInter = LAZY_ROPE_INTERLEAVED, kvAlibi = LAZY_ALIBI };

// cos/sin for pairs k = 8c .. 8c+7 at position pos
template <int DH>
__device__ __forceinline__ void pair_coefs(const KvArgs& a, int pos, int c, float (&cs)[8], float (&sn)[8]) {
  if (a.cos_sin != nullptr) {
    const float* row = a.cos_sin + (int64_t)pos * DH + 8 * c;
    const f32x4 c0 = *reinterpret_cast<const f32x4*>(row);
    const f32x4 c1 = *reinterpret_cast<const f32x4*>(row + 4);
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(row + DH / 2);
    const f32x4 s1 = *reinterpret_cast<const f32x4*>(row + DH / 2 + 4);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      cs[t] = c0[t];
      cs[4 + t] = c1[t];
      sn[t] = s0[t];
      sn[4 + t] = s1[t];
    }
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      sincos_reduced(pos, a.inv_freq[8 * c + t], &sn[t], &cs[t]);
    }
  }
}

// Rotate (KIND != ALiBi) the 16 channels of a row owned by chunk c: reads src, writes dst.
template <typename T, int DH, int KIND>
__device__ __forceinline__ void rotate_row(const KvArgs& a, const T* src, T* dst, int pos, int c) {
  using E = Elem<T>;
  using F8 = typename E::Frag8;
  if (KIND == kvAlibi) {
    const F8 x0 = load8<T>(src + 16 * c), x1 = load8<T>(src + 16 * c + 8);
    *reinterpret_cast<F8*>(dst + 16 * c) = x0;
    *reinterpret_cast<F8*>(dst + 16 * c + 8) = x1;
    return;
  }
  float cs[8], sn[8];
  pair_coefs<DH>(a, pos, c, cs, sn);
  if (KIND == kvHalf) {
    // pairs (8c + t, dh/2 + 8c + t)
    const F8 lo = load8<T>(src + 8 * c), hi = load8<T>(src + DH / 2 + 8 * c);
    F8 olo, ohi;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float x1 = E::to_f(lo[t]), x2 = E::to_f(hi[t]);
      olo[t] = E::from_f(x1 * cs[t] - x2 * sn[t]);
      ohi[t] = E::from_f(x1 * sn[t] + x2 * cs[t]);
    }
    *reinterpret_cast<F8*>(dst + 8 * c) = olo;
    *reinterpret_cast<F8*>(dst + DH / 2 + 8 * c) = ohi;
  } else {
    // pairs (2k, 2k + 1), k = 8c + t: channels 16c .. 16c + 15
    const F8 x0 = load8<T>(src + 16 * c), x1 = load8<T>(src + 16 * c + 8);
    F8 o0, o1;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float a1 = E::to_f(x0[2 * t]), a2 = E::to_f(x0[2 * t + 1]);
      o0[2 * t] = E::from_f(a1 * cs[t] - a2 * sn[t]);
      o0[2 * t + 1] = E::from_f(a1 * sn[t] + a2 * cs[t]);
      const float b1 = E::to_f(x1[2 * t]), b2 = E::to_f(x1[2 * t + 1]);
      o1[2 * t] = E::from_f(b1 * cs[4 + t] - b2 * sn[4 + t]);
      o1[2 * t + 1] = E::from_f(b1 * sn[4 + t] + b2 * cs[4 + t]);
    }
    *reinterpret_cast<F8*>(dst + 16 * c) = o0;
    *reinterpret_cast<F8*>(dst + 16 * c + 8) = o1;
  }
}

// The channels rotate_row writes for chunk c, set to NaN (a token whose
// rotation position is invalid: its row must not pass for a rotated one).
template <typename T, int DH, int KIND>
__device__ __forceinline__ void poison_row(T* dst, int c) {
  using F8 = typename Elem<T>::Frag8;
  F8 nan;
#pragma unroll
  for (int t = 0; t < 8; ++t) nan[t] = Elem<T>::from_f(__builtin_nanf(""));
  if (KIND == kvHalf) {
    *reinterpret_cast<F8*>(dst + 8 * c) = nan;
    *reinterpret_cast<F8*>(dst + DH / 2 + 8 * c) = nan;
  } else {
    *reinterpret_cast<F8*>(dst + 16 * c) = nan;
    *reinterpret_cast<F8*>(dst + 16 * c + 8) = nan;
  }
}

// blockIdx.y: 0 = K rows, 1 = V rows, 2 = Q rows
template <typename T, int DH, int KIND>
__global__ __launch_bounds__(256) void kv_write_kernel(KvArgs a) {
  constexpr int CPR = DH / 16;  // chunks (threads) per row
  const int which = blockIdx.y;
  const int heads = (which == 2) ? a.hq : a.hkv;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t items = (int64_t)a.num_tokens * heads * CPR;
  if (idx >= items) return;
  const int c = (int)(idx % CPR);
  const int h = (int)((idx / CPR) % heads);
  const int t = (int)(idx / ((int64_t)CPR * heads));

  const int pos = a.positions[t];
  // a rotation position the coefficients cannot serve (negative, or past the
  // table): the token's rows become NaN instead of being skipped, so the
  // mistake surfaces in every output that reads them
  const bool bad_pos = KIND != kvAlibi && (pos < 0 || (a.cos_sin != nullptr && pos >= a.max_pos));

  if (which == 2) {
    T* row = reinterpret_cast<T*>(a.q) + ((int64_t)t * a.hq + h) * DH;
    if (bad_pos)
      poison_row<T, DH, KIND>(row, c);
    else if (KIND != kvAlibi)
      rotate_row<T, DH, KIND>(a, row, row, pos, c);
    return;
  }
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= a.num_slots) return;  // never write outside the pool
  const int64_t blk = slot / kBlock;
  const int s = (int)(slot % kBlock);
  const int64_t base = (blk * a.hkv + h) * (int64_t)(kBlock * DH);
  if (which == 0) {
    const T* src = reinterpret_cast<const T*>(a.k) + ((int64_t)t * a.hkv + h) * DH;
    T* dst = reinterpret_cast<T*>(a.k_cache) + base + (int64_t)s * DH;
    if (bad_pos)
      poison_row<T, DH, KIND>(dst, c);
    else
      rotate_row<T, DH, KIND>(a, src, dst, pos, c);
  } else {
    const T* src = reinterpret_cast<const T*>(a.v) + ((int64_t)t * a.hkv + h) * DH + 16 * c;
    T* dst = reinterpret_cast<T*>(a.v_cache) + base + (int64_t)(16 * c) * kBlock + s;
    const typename Elem<T>::Frag8 x0 = load8<T>(src), x1 = load8<T>(src + 8);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      dst[d * kBlock] = x0[d];
      dst[(8 + d) * kBlock] = x1[d];
    }
  }
}

namespace {

template <typename T, int DH>
hipError_t launch_kv(int kind, const KvArgs& a, bool with_q, hipStream_t st) {
  const int ys = with_q ? 3 : 2;
  const int64_t items = (int64_t)a.num_tokens * (with_q ? std::max(a.hq, a.hkv) : a.hkv) * (DH / 16);
  dim3 grid((unsigned)((items + 255) / 256), (unsigned)ys);
  switch (kind) {
    case kvHalf:
      hipLaunchKernelGGL((kv_write_kernel<T, DH, kvHalf>), grid, dim3(256), 0, st, a);
      break;
    case kvInter:
      hipLaunchKernelGGL((kv_write_kernel<T, DH, kvInter>), grid, dim3(256), 0, st, a);
      break;
    default:
      hipLaunchKernelGGL((kv_write_kernel<T, DH, kvAlibi>), grid, dim3(256), 0, st, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace
}  // namespace lazy

using namespace lazy;

extern "C" lazy_status lazy_kv_write(const lazy_geom* geom, const lazy_pos_desc* pos, void* k_cache, void* v_cache,
                                     int64_t num_blocks, const void* k, const void* v, void* q_inout,
                                     const int32_t* positions, const int64_t* slot_mapping, int32_t num_tokens,
                                     void* stream) {
  clear_error();
  lazy_status st = check_geom(geom);
  if (st != LAZY_OK) return st;
  st = check_pos(geom, pos);
  if (st != LAZY_OK) return st;
  if (num_tokens < 0) return fail(LAZY_ERR_ARG, "num_tokens must be >= 0");
  if (num_blocks < 1 || num_blocks > (int64_t)LAZY_MAX_BLOCK_ID + 1)
    return fail(LAZY_ERR_ARG, "num_blocks must be in [1, 2^24]");
  if (num_tokens == 0) return LAZY_OK;
  if (!k_cache || !v_cache || !k || !v || !positions || !slot_mapping)
    return fail(LAZY_ERR_ARG, "a required device pointer is NULL");
  if ((int64_t)num_tokens * std::max(geom->num_q_heads, geom->num_kv_heads) * (geom->head_dim / 16) >
      (int64_t)65535 * 256 * 1024)
    return fail(LAZY_ERR_UNSUPPORTED, "too many tokens in one call");
  KvArgs a{};
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_slots = num_blocks * kBlock;
  a.k = k;
  a.v = v;
  a.q = q_inout;
  a.positions = positions;
  a.slots = slot_mapping;
  a.cos_sin = pos->cos_sin;
  a.inv_freq = pos->inv_freq;
  a.max_pos = pos->max_pos;
  a.num_tokens = num_tokens;
  a.hq = geom->num_q_heads;
  a.hkv = geom->num_kv_heads;
  // q only needs work under RoPE
  const bool with_q = q_inout != nullptr && pos->kind != LAZY_ALIBI;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (geom->dtype == LAZY_BF16)
    e = geom->head_dim == 128 ? launch_kv<bf16, 128>(pos->kind, a, with_q, s) : launch_kv<bf16, 64>(pos->kind, a, with_q, s);
  else
    e = geom->head_dim == 128 ? launch_kv<float, 128>(pos->kind, a, with_q, s)
                              : launch_kv<float, 64>(pos->kind, a, with_q, s);
  if (e != hipSuccess) return fail(LAZY_ERR_HIP, "kv write launch failed: %s", hipGetErrorString(e));
  return LAZY_OK;
}
