// fa_splitkv.hip -- split-KV attention forward for decode (few queries, long key
// sequences) on gfx950 (MI355X), and its C ABI.
//
// The reference lists of the pages name work-centric and split schedules for decoding
// (the Lean Attention and Stream-K titles) without describing them. Here the key axis of
// every (batch, K/V head) is cut into S ranges; each range is one independent unit of
// work that leaves a partial output normalised over its own keys and the log-sum-exp of
// its scores, and a merge kernel combines the S partials exactly:
//     lse = ln sum_s exp(lse_s),   O = sum_s exp(lse_s - lse) O_s
// (the split identity that the oracle's pins check). The Nq queries are the last Nq
// positions of the sequence; under the causal mask query i sees keys j <= Nk - Nq + i.
//
// gfx950 mapping. Decode is bound by reading K and V from HBM, so the design keeps every
// wavefront streaming: one wavefront per unit, four independent wavefronts per workgroup
// (no barriers), all the query rows of the K/V head's group (group x Nq <= 64) packed as
// the columns of S^T = K Q^T on v_mfma_f32_32x32x16, so each K/V element read from HBM
// serves every query head that shares it. Each 32-key block is read with whole rows per
// load instruction (fully used cache lines) into a per-wavefront LDS tile: K row-major
// with a 16-byte-chunk swizzle, from which the S^T operands are read; V row-major, from
// which ds_read_b64_tr_b16 reads the V^T operands of O^T += V^T P^T already transposed.
// The next block's loads are in flight while the current one is computed. The online
// softmax is lane-local (one query row per lane pair).
#include <hip/hip_runtime.h>

#include <mutex>

#include <cmath>
#include <cstdint>

#include "fa.h"
#include "fa_env.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;          // 4 independent wavefronts
constexpr int kBlk = 32;               // keys per block
constexpr float kLn2 = 0.6931471805599453f;

struct Bf16 {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned pack2(float x, float y) {
    bf16x2 r = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(unsigned, r);
  }
};
struct F16 {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned pack2(float x, float y) {
    f16x2 r = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(unsigned, r);
  }
};

struct SkvArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* part_o;         // workspace: [S][B][H][Nq][D], each normalised over its keys
  float* part_lse;       // workspace: [S][B][H][Nq]
  int B, H, Hkv, Nq, Nk, group;
  int S;                 // key ranges per (batch, K/V head)
  int L;                 // keys per range (a multiple of kBlk)
  int rows;              // group * Nq query rows per (batch, K/V head)
  int units;             // B * Hkv * S
  float c;               // scale * log2(e)
};

// Per-wavefront LDS tiles of one 32-key block, both row-major (key rows of 2D bytes):
//   K: 16-byte chunk c of row r at chunk position c ^ kswz(r), so that the 32 lanes reading
//      one chunk of 32 consecutive rows (the S^T operand) spread over the banks;
//   V: 32-byte segment s of row r at segment s ^ (r & 3), so that the 4 rows of one
//      transposing read (ds_read_b64_tr_b16) fall on different banks.
template <int D>
__device__ __forceinline__ int kswz(int r) {
  if constexpr (D == 128) {
    const int x = r & 3;
    return ((x << 1) ^ (x << 2)) ^ ((r >> 2) & 3);
  } else {
    return r & 7;
  }
}
template <int D>
__device__ __forceinline__ int kt_byte(int r, int chunk) {
  return r * (2 * D) + ((chunk ^ kswz<D>(r)) << 4);
}
template <int D>
__device__ __forceinline__ int vt_byte(int r, int byte) {     // byte offset inside the row
  return r * (2 * D) + (byte ^ ((r & 3) << 5));
}
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_byte;

template <typename Ops, int D, int RB, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void splitkv_partial_kernel(SkvArgs a) {
  constexpr int kKsteps = D / 16;
  constexpr int kDblocks = D / 32;
  constexpr int kChunks = D / 8;           // 16-byte chunks per row
  constexpr int kRowsLd = 64 / kChunks;     // rows per wavefront load
  constexpr int kLds = kBlk / kRowsLd;      // loads per tensor per block
  constexpr int kTile = kBlk * D * 2;       // one 32-key tile
  __shared__ __attribute__((aligned(16))) unsigned char lds[4 * 2 * kTile];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int unit = blockIdx.x * 4 + wave;
  if (unit >= a.units) return;             // whole wavefront; the kernel has no barriers
  unsigned char* kt = lds + wave * (2 * kTile);   // this wavefront's K tile, then its V tile
  unsigned char* vt = kt + kTile;
  const int s = unit % a.S;
  const int bh = unit / a.S;               // b * Hkv + hk
  const int hk = bh % a.Hkv, b = bh / a.Hkv;
  const int Nk = a.Nk, Nq = a.Nq;
  const int j_begin = s * a.L;
  const int j_end = min(Nk, j_begin + a.L);

  // query rows of this lane (MFMA column l32 of each 32-row block): row r -> head
  // hk*group + r / Nq, query r % Nq at sequence position Nk - Nq + r % Nq
  u32x4 qreg[RB][kKsteps];
  int qpos[RB];
  bool qvalid[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = rb * 32 + l32;
    qvalid[rb] = r < a.rows;
    const int rr = qvalid[rb] ? r : 0;
    const int h = hk * a.group + rr / Nq, i = rr % Nq;
    qpos[rb] = Nk - Nq + i;
    const uint16_t* qp = (const uint16_t*)a.q + (((size_t)b * Nq + i) * a.H + h) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < kKsteps; ++ks) qreg[rb][ks] = *(const u32x4*)(qp + 16 * ks);
  }

  f32x16 oacc[RB][kDblocks];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < kDblocks; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[rb][i][e] = 0.0f;
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -__FLT_MAX__;              // finite, so that exp2(-inf - m) = 0, never NaN
    l_run[rb] = 0.0f;
  }

  const size_t kv_row = (size_t)a.Hkv * D;
  const uint16_t* kbase = (const uint16_t*)a.k + (size_t)b * Nk * kv_row + (size_t)hk * D;
  const uint16_t* vbase = (const uint16_t*)a.v + (size_t)b * Nk * kv_row + (size_t)hk * D;

  // K and V of one block, whole rows per load (lane: row u*kRowsLd + lane/kChunks, chunk
  // lane%kChunks); the next block's loads go out as soon as these registers are in LDS,
  // so they are in flight during S^T, the softmax and the P.V products
  const int ld_row = lane / kChunks, ld_chunk = lane % kChunks;
  u32x4 kn[kLds], vn[kLds];
  auto load = [&](int jb) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kLds; ++u) {
      const size_t r = (size_t)min(jb + u * kRowsLd + ld_row, Nk - 1);
      kn[u] = *(const u32x4*)(kbase + r * kv_row + 8 * ld_chunk);
      vn[u] = *(const u32x4*)(vbase + r * kv_row + 8 * ld_chunk);
    }
  };
  if (j_begin < j_end) load(j_begin);

  // V^T operand of the P.V MFMA for k-step t2 and dim block db: for k index 8hi + i the
  // P^T operand holds key 16t2 + 8(i/4) + 4hi + i%4, so elements 0-3 and 4-7 are 4
  // consecutive keys each, one transposing read apiece (lane j of a 16-lane group gets
  // dim dbase + j of 4 rows; lane 4r + c supplies row r's dims dbase + 4c .. +3)
  const int tr_row = (lane & 15) >> 2, tr_col = 8 * (lane & 3) + 32 * ((lane >> 4) & 1);   // bytes
  auto vt_operand = [&](int t2, int db) __attribute__((always_inline)) {
    const int r1 = 16 * t2 + 4 * hi + tr_row, r2 = r1 + 8;
    const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)((lds_byte*)vt + vt_byte<D>(r1, 64 * db + tr_col)));
    const s16x4 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)((lds_byte*)vt + vt_byte<D>(r2, 64 * db + tr_col)));
    const u32x2 w1 = __builtin_bit_cast(u32x2, x1), w2 = __builtin_bit_cast(u32x2, x2);
    return u32x4{w1[0], w1[1], w2[0], w2[1]};
  };

  for (int jb = j_begin; jb < j_end; jb += kBlk) {
#pragma unroll
    for (int u = 0; u < kLds; ++u) {
      const int r = u * kRowsLd + ld_row;
      *(u32x4*)(kt + kt_byte<D>(r, ld_chunk)) = kn[u];
      *(u32x4*)(vt + vt_byte<D>(r, 16 * ld_chunk)) = vn[u];
    }
    if (jb + kBlk < j_end) load(jb + kBlk);
    f32x16 st[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) st[rb][e] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < kKsteps; ++ks)
        st[rb] = Ops::mfma(*(const u32x4*)(kt + kt_byte<D>(l32, 2 * ks + hi)), qreg[rb][ks], st[rb]);
    }

#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      // mask: keys past the range or the sequence, and (causal) past the query's position
      const bool need_mask = jb + kBlk > j_end || (CAUSAL && jb + kBlk - 1 > Nk - Nq);
      if (need_mask) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = jb + 8 * (e >> 2) + 4 * hi + (e & 3);
          const bool dead = key >= j_end || (CAUSAL && key > qpos[rb]);
          st[rb][e] = dead ? -INFINITY : st[rb][e];
        }
      }
      float mx = st[rb][0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, st[rb][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));             // the row's other 16 keys
      const float m_new = fmaxf(m_run[rb], mx * a.c);
      const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - m_new);
      m_run[rb] = m_new;
      float p[16], sum = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[rb][e], a.c, -m_new));
        sum += p[e];
      }
      l_run[rb] = l_run[rb] * alpha + sum;
#pragma unroll
      for (int i = 0; i < kDblocks; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[rb][i][e] *= alpha;
      u32x4 pb[2];
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int w = 0; w < 4; ++w) pb[t2][w] = Ops::pack2(p[8 * t2 + 2 * w], p[8 * t2 + 2 * w + 1]);
      // O^T += V^T P^T: A = V^T rows (dims 32 db + l32), slots 16 t2 + 8 hi .. +7
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int db = 0; db < kDblocks; ++db) {
          oacc[rb][db] = Ops::mfma(vt_operand(t2, db), pb[t2], oacc[rb][db]);
        }
    }
  }

  // partial outputs of this range, normalised over its keys
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l_tot = l_run[rb] + __shfl_xor(l_run[rb], 32, 64);
    if (!qvalid[rb]) continue;
    const int r = rb * 32 + l32;
    const int h = hk * a.group + r / Nq, i = r % Nq;
    const size_t prow = (((size_t)s * a.B + b) * a.H + h) * Nq + i;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    float* po = a.part_o + prow * D;
#pragma unroll
    for (int db = 0; db < kDblocks; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 w;
        w.x = oacc[rb][db][4 * g] * inv;
        w.y = oacc[rb][db][4 * g + 1] * inv;
        w.z = oacc[rb][db][4 * g + 2] * inv;
        w.w = oacc[rb][db][4 * g + 3] * inv;
        *(float4*)(po + 32 * db + 8 * g + 4 * hi) = w;
      }
    if (hi == 0) a.part_lse[prow] = l_tot > 0.0f ? (m_run[rb] + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
  }
}

// merge: one row (b, h, i) per 64 lanes, D/64 dims per lane
template <typename Ops, int D>
__global__ __launch_bounds__(kThreads) void splitkv_merge_kernel(SkvArgs a) {
  constexpr int kPer = D / 64;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);   // (b, h, i), i fastest
  const int lane = threadIdx.x & 63;
  const int nrows = a.B * a.H * a.Nq;
  if (row >= nrows) return;
  const size_t plane = (size_t)nrows;                    // rows per split
  // the loops over the ranges are unrolled so that several ranges' loads are in flight
  // at once (one range at a time left the kernel waiting on one load latency per range)
  float m = -INFINITY;
#pragma unroll 8
  for (int s = 0; s < a.S; ++s) m = fmaxf(m, a.part_lse[s * plane + row]);
  float w_sum = 0.0f;
  float acc[kPer];
#pragma unroll
  for (int t = 0; t < kPer; ++t) acc[t] = 0.0f;
#pragma unroll 8
  for (int s = 0; s < a.S; ++s) {
    const float ls = a.part_lse[s * plane + row];
    const float w = ls == -INFINITY ? 0.0f : __expf(ls - m);
    w_sum += w;
    const float* po = a.part_o + (s * plane + row) * D + lane * kPer;
#pragma unroll
    for (int t = 0; t < kPer; ++t) acc[t] += w * po[t];
  }
  const float inv = 1.0f / w_sum;
  const int i = row % a.Nq, h = (row / a.Nq) % a.H, b = row / (a.Nq * a.H);
  uint16_t* op = (uint16_t*)a.o + (((size_t)b * a.Nq + i) * a.H + h) * D + lane * kPer;
  if constexpr (kPer == 2) {
    *(unsigned*)op = Ops::pack2(acc[0] * inv, acc[1] * inv);
  } else {
    const unsigned w = Ops::pack2(acc[0] * inv, 0.0f);
    *op = (uint16_t)(w & 0xffffu);
  }
  if (lane == 0) a.lse[((size_t)b * a.H + h) * a.Nq + i] = m + __logf(w_sum);
}

// ---- host ----------------------------------------------------------------------------
bool aligned(const void* p, size_t n) { return ((uintptr_t)p % n) == 0; }

// Ranges per (batch, K/V head): num_splits if positive, else about one unit per SIMD
// (1024 on MI355X; the d = 128 kernel holds one wavefront per SIMD, so more units only
// queue behind the first round) with at least 256 keys each; then the range length is
// rounded up to whole key blocks and the count recomputed, so that no range is empty.
void plan(int B, int Hkv, int Nk, int num_splits, int* S, int* L) {
  int s = num_splits;
  if (s <= 0) {
    const int want = (1024 + B * Hkv - 1) / (B * Hkv);
    const int most = (Nk + 255) / 256;
    s = want < most ? want : most;
  }
  if (s < 1) s = 1;
  if (s > Nk) s = Nk;
  int len = (Nk + s - 1) / s;
  len = (len + kBlk - 1) / kBlk * kBlk;
  *L = len;
  *S = (Nk + len - 1) / len;
}

fa_status check_splitkv(int B, int H, int Hkv, int Nq, int Nk, int d, int causal, fa_dtype dtype) {
  if (B < 1 || H < 1 || Hkv < 1 || Nq < 1 || Nk < Nq || d < 1) return FA_ERR_INVALID_ARG;
  if (Hkv > H || H % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) {
    return dtype == FA_DTYPE_FP8_E4M3 ? FA_ERR_UNSUPPORTED : FA_ERR_INVALID_ARG;
  }
  if ((long long)B * Nk * Hkv * d >= (1LL << 31) || (long long)B * Nq * H * d >= (1LL << 31)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((long long)(H / Hkv) * Nq > 64) return FA_ERR_UNSUPPORTED;   // query rows per K/V head
  return FA_OK;
}

template <typename Ops, int D, int RB, bool CAUSAL>
fa_status launch_partial(const SkvArgs& args, hipStream_t s) {
  fa_env::log_launch("splitkv_partial_kernel", __PRETTY_FUNCTION__, (args.units + 3) / 4, kThreads);
  hipLaunchKernelGGL((splitkv_partial_kernel<Ops, D, RB, CAUSAL>), dim3((args.units + 3) / 4), dim3(kThreads), 0, s, args);
  if (hipGetLastError() != hipSuccess) return FA_ERR_LAUNCH;
  const int rows = args.B * args.H * args.Nq;
  fa_env::log_launch("splitkv_merge_kernel", __PRETTY_FUNCTION__, (rows + 3) / 4, kThreads);
  hipLaunchKernelGGL((splitkv_merge_kernel<Ops, D>), dim3((rows + 3) / 4), dim3(kThreads), 0, s, args);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

template <typename Ops, int D>
fa_status dispatch_rb(const SkvArgs& args, int causal, hipStream_t s) {
  if (args.rows <= 32) return causal ? launch_partial<Ops, D, 1, true>(args, s) : launch_partial<Ops, D, 1, false>(args, s);
  return causal ? launch_partial<Ops, D, 2, true>(args, s) : launch_partial<Ops, D, 2, false>(args, s);
}

// The workspace of one call: every partial output and lse is written by the partial kernel
// before the merge kernel reads it, so the buffer's previous contents never matter.
size_t splitkv_bytes(int B, int H, int Nq, int d, int S) { return (size_t)S * B * H * Nq * (d + 1) * sizeof(float); }

fa_status splitkv_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv,
                       int Nq, int Nk, int d, int causal, float scale, fa_dtype dtype, int num_splits,
                       float* workspace, size_t workspace_bytes, hipStream_t s) {
  SkvArgs args;
  plan(B, Hkv, Nk, num_splits, &args.S, &args.L);
  if (workspace_bytes < splitkv_bytes(B, H, Nq, d, args.S)) return FA_ERR_INVALID_ARG;
  if ((long long)B * Hkv * args.S > 0x7fffffffLL - 3) return FA_ERR_INVALID_ARG;
  args.q = q;
  args.k = k;
  args.v = v;
  args.o = o;
  args.lse = lse;
  args.part_o = workspace;
  args.part_lse = workspace + (size_t)args.S * B * H * Nq * d;
  args.B = B;
  args.H = H;
  args.Hkv = Hkv;
  args.Nq = Nq;
  args.Nk = Nk;
  args.group = H / Hkv;
  args.rows = args.group * Nq;
  args.units = B * Hkv * args.S;
  args.c = (float)((double)scale * 1.4426950408889634);
  if (dtype == FA_DTYPE_BF16) return d == 128 ? dispatch_rb<Bf16, 128>(args, causal, s) : dispatch_rb<Bf16, 64>(args, causal, s);
  return d == 128 ? dispatch_rb<F16, 128>(args, causal, s) : dispatch_rb<F16, 64>(args, causal, s);
}

fa_status splitkv_checks(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv,
                         int Nq, int Nk, int d, int causal, float scale, fa_dtype dtype) {
  fa_status st = check_splitkv(B, H, Hkv, Nq, Nk, d, causal, dtype);
  if (st != FA_OK) return st;
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 4) || !aligned(lse, 4))
    return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

// Library-owned scratch for fa_fwd_splitkv_static: one copy of this array per GPU, held
// until the process ends. Host code never passes the array's name to a kernel (in host
// code it is a host-side stand-in, not a device address); it uses the device address that
// hipGetSymbolAddress returns on each device, looked up once per device on that device's
// first call.
constexpr size_t kStaticScratchBytes = FA_SPLITKV_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// this device's address of `scratch` (nullptr if the lookup failed)
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t fa_fwd_splitkv_workspace_bytes(int B, int H, int Hkv, int Nq, int Nk, int d, int num_splits) {
  if (B < 1 || H < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || d < 1) return 0;
  int S, L;
  plan(B, Hkv, Nk, num_splits, &S, &L);
  return splitkv_bytes(B, H, Nq, d, S);
}

fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                         int Hkv, int Nq, int Nk, int d, int causal, float scale, fa_dtype dtype,
                         int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  fa_status st = splitkv_checks(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, causal, scale, dtype);
  if (st != FA_OK) return st;
  if (!workspace || !aligned(workspace, 16)) return FA_ERR_INVALID_ARG;
  return splitkv_impl(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, causal, scale, dtype, num_splits, (float*)workspace,
                      workspace_bytes, (hipStream_t)stream);
}

fa_status fa_fwd_splitkv_static(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                int Hkv, int Nq, int Nk, int d, int causal, float scale, fa_dtype dtype,
                                int num_splits, void* stream) {
  fa_status st = splitkv_checks(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, causal, scale, dtype);
  if (st != FA_OK) return st;
  int S, L;
  plan(B, Hkv, Nk, num_splits, &S, &L);
  if (splitkv_bytes(B, H, Nq, d, S) > kStaticScratchBytes) return FA_ERR_SCRATCH;
  void* ws = scratch_on_current_device();
  if (!ws) return FA_ERR_LAUNCH;
  return splitkv_impl(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, causal, scale, dtype, num_splits, (float*)ws,
                      kStaticScratchBytes, (hipStream_t)stream);
}

}  // extern "C"
