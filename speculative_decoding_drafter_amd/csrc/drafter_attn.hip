// drafter_attn.hip -- gfx950 (CDNA4) kernels and C ABI for the DFlash drafter's
// block attention (TensorRT-LLM PR #20532, commits adding k3_drafter_attn /
// k3_drafter_attn_qknorm and their contracts).  The ABI is documented in
// include/drafter_attn.h.
//
// One launch per call.  Workgroup (split s, KV head g, request r), 4 waves:
//   1. prologue: the 6*T query rows of group g (and, in the last split, the
//      block's own K/V rows) go to LDS as bf16; in the qknorm variant each row
//      is RMS-normalised and NeoX-rotated in fp32 on the way (angle in fp64).
//   2. page loop: wave w walks pages s*Ps+w, +4, ... of the split.  Per page:
//      K rows are loaded straight into MFMA A-fragments, S^T = K.Q^T with
//      v_mfma_f32_16x16x32_bf16, online softmax in the exp2 domain, V is
//      transposed through a per-wave LDS tile, O^T += V^T.P^T with MFMA.  The
//      next page's K/V loads are in flight while the current page computes.
//   3. the 4 waves merge (max, sum, output) through LDS and write one fp32
//      partial per workgroup;
//   4. the last workgroup of each (r, g) (device-scope counter, reset by that
//      workgroup) merges the splits in fixed order and writes bf16 output.
// Nothing depends on device data except through loads, so the same launch is
// valid for any rewritten lengths / page tables / qkv (graph replay), and the
// split plan and every reduction order are fixed (bit-identical reruns).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <string>

#include "drafter_attn.h"

namespace {

constexpr int kD = 64;        // head_dim
constexpr int kPage = 64;     // tokens per page
constexpr int kG = 6;         // query heads per KV head
constexpr int kMaxT = 8;      // tokens per block
constexpr int kRows = 48;     // kG * kMaxT query rows per workgroup
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxSplits = 64;
constexpr int kTileBytes = kPage * kD * 2;   // one [64][64] bf16 tile, 8 KiB

// LDS layout (bytes)
constexpr int kOffQ = 0;                                   // [48][64] bf16 query tile
constexpr int kOffCS = kOffQ + kRows * kD * 2;             // [8][32] (cos, sin) fp32
constexpr int kOffMW = kOffCS + kMaxT * 32 * 8;            // [4][48] per-wave running max
constexpr int kOffLW = kOffMW + kWaves * kRows * 4;        // [4][48] per-wave weight sum
constexpr int kOffFlag = kOffLW + kWaves * kRows * 4;      // last-workgroup flag
constexpr int kOffU = kOffFlag + 16;                       // union region
constexpr int kOffVT = kOffU;                              // [4 waves] V^T tiles
constexpr int kOffKown = kOffVT + kWaves * kTileBytes;     // own-block K tile
constexpr int kOffVown = kOffKown + kTileBytes;            // own-block V tile
constexpr int kObufStride = kD + 4;                        // fp32 row stride (pad: no bank conflicts)
constexpr int kOffObuf = kOffU;                            // [4][48][68] fp32 merge buffer
constexpr int kOffWts = kOffU;                             // [kMaxSplits][48] fp32 combine weights
constexpr int kUnionBytes = (kWaves * kRows * kObufStride * 4 > kWaves * kTileBytes + 2 * kTileBytes)
                                ? kWaves * kRows * kObufStride * 4
                                : kWaves * kTileBytes + 2 * kTileBytes;
constexpr int kSmemBytes = kOffU + kUnionBytes;
static_assert(kMaxSplits * kRows * 4 <= kUnionBytes, "combine weights must fit the union");
static_assert(kSmemBytes <= 64 * 1024, "LDS budget");

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Params {
  const uint16_t* qkv;
  int64_t qkv_stride;
  const uint16_t* kpool;
  const uint16_t* vpool;
  int64_t page_stride;
  const int32_t* page_table;
  const int32_t* ctx_lens;
  const int32_t* blk_lens;
  const void* positions;
  const uint16_t* wq;
  const uint16_t* wk;
  float* part_o;     // [R*Hkv*S][48][64]
  float* part_ml;    // [R*Hkv*S][48][2]
  uint32_t* counters;  // [R*Hkv]
  uint16_t* out;
  int64_t out_stride;
  int32_t* status;
  int32_t num_pages;
  int32_t pt_stride;
  int32_t R, T, Hq, Hkv;
  int32_t S, Ps;
  float c;    // scale * log2(e): scores live in the exp2 domain
  float eps;
  double log2_base;  // log2(rope_base), fp64
};

// ---------------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------------

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (gfx950 converts in hardware)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = static_cast<__bf16>(lo);
  __bf16 b = static_cast<__bf16>(hi);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// XOR swizzle of the 16-byte chunk inside a 128-byte LDS row: keeps both the
// transposing writes (8 rows 8 apart) and the fragment reads (8 consecutive
// rows) on distinct banks.
__device__ __forceinline__ int swz(int row) { return ((row >> 3) ^ row) & 7; }

__device__ __forceinline__ int tile_off(int row, int chunk) {
  return row * (kD * 2) + ((chunk ^ swz(row)) << 4);
}

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The key a lane's A-fragment row / S^T output register stands for.  The 64
// keys of a page are permuted so that (a) the P^T registers a lane owns after
// the score MFMA are exactly the B-fragment of the PV MFMA and (b) the V^T
// fragment a lane needs is one contiguous 16-byte LDS chunk.  `mt` = 16-key
// M-tile, `r16` = row inside the tile.
__device__ __forceinline__ int key_of(int mt, int r16) {
  return 32 * (mt & 1) + 8 * (r16 & 3) + 4 * (mt >> 1) + (r16 >> 2);
}

struct KFrag { u32x4 a[4][2]; };   // [M-tile][k-step]: K rows in A-fragment layout
struct VFrag { u32x4 v[8]; };      // [jj]: key 8*jj + lane/8, dims 8*(lane%8) .. +7

__device__ __forceinline__ void load_k_global(KFrag& k, const uint16_t* base, int lane) {
  const int r16 = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const uint16_t* row = base + key_of(mt, r16) * kD + 8 * lg;
    k.a[mt][0] = ld16(row);
    k.a[mt][1] = ld16(row + 32);
  }
}

__device__ __forceinline__ void load_v_global(VFrag& v, const uint16_t* base, int lane) {
  const uint16_t* p = base + (lane >> 3) * kD + 8 * (lane & 7);
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) v.v[jj] = ld16(p + jj * 8 * kD);
}

__device__ __forceinline__ void load_k_lds(KFrag& k, const unsigned char* tile, int lane) {
  const int r16 = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int row = key_of(mt, r16);
    k.a[mt][0] = *reinterpret_cast<const u32x4*>(tile + tile_off(row, lg));
    k.a[mt][1] = *reinterpret_cast<const u32x4*>(tile + tile_off(row, 4 + lg));
  }
}

__device__ __forceinline__ void load_v_lds(VFrag& v, const unsigned char* tile, int lane) {
#pragma unroll
  for (int jj = 0; jj < 8; ++jj)
    v.v[jj] = *reinterpret_cast<const u32x4*>(tile + tile_off(8 * jj + (lane >> 3), lane & 7));
}

// ---------------------------------------------------------------------------------
// one page (64 keys) of online-softmax attention for one wave, 16*NT query rows
// ---------------------------------------------------------------------------------
template <int NT, bool TAIL>
__device__ __forceinline__ void attend_page(const KFrag& k, VFrag& v, int valid,
                                            const u32x4 (&qf)[NT][2], f32x4 (&o)[NT][4],
                                            float (&m_run)[NT], float (&l_run)[NT], float c,
                                            unsigned char* vt, int lane) {
  const int lg = lane >> 4;
  // ---- S^T = K . Q^T  (rows: keys, cols: query rows)
  f32x4 s[NT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma(k.a[mt][0], qf[nt][0], acc);
      acc = mfma(k.a[mt][1], qf[nt][1], acc);
      s[nt][mt] = acc;
    }
  if (TAIL) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 32 * (mt & 1) + 8 * i + 4 * (mt >> 1) + lg;
        if (key >= valid) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) s[nt][mt][i] = -INFINITY;
        }
      }
  }
  // ---- online softmax per query column (lane & 15), exp2 domain
  u32x4 pf[NT][2];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float mx = s[nt][0][0];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[nt][mt][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run[nt], mx);
    const float alpha = fast_exp2((m_run[nt] - m_new) * c);
    m_run[nt] = m_new;
    const float nmc = -m_new * c;
    float p[4][4];
    float lsum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[mt][i] = fast_exp2(fmaf(s[nt][mt][i], c, nmc));
        lsum += p[mt][i];
      }
    l_run[nt] = fmaf(l_run[nt], alpha, lsum);
#pragma unroll
    for (int md = 0; md < 4; ++md) o[nt][md] *= alpha;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      pf[nt][ks][0] = pack_bf16x2(p[2 * ks][0], p[2 * ks][1]);
      pf[nt][ks][1] = pack_bf16x2(p[2 * ks][2], p[2 * ks][3]);
      pf[nt][ks][2] = pack_bf16x2(p[2 * ks + 1][0], p[2 * ks + 1][1]);
      pf[nt][ks][3] = pack_bf16x2(p[2 * ks + 1][2], p[2 * ks + 1][3]);
    }
  }
  // ---- V^T through this wave's LDS tile
  const int cgrp = lane >> 3, u = lane & 7;
  if (TAIL) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      if (8 * jj + cgrp >= valid) v.v[jj] = u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    u32x4 w;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = __builtin_amdgcn_perm(v.v[2 * q + 1][e >> 1], v.v[2 * q][e >> 1], sel);
    *reinterpret_cast<u32x4*>(vt + tile_off(8 * u + e, cgrp)) = w;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int md = 0; md < 4; ++md) {
    const int d = 16 * md + (lane & 15);
    const u32x4 a0 = *reinterpret_cast<const u32x4*>(vt + tile_off(d, lg));
    const u32x4 a1 = *reinterpret_cast<const u32x4*>(vt + tile_off(d, 4 + lg));
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      o[nt][md] = mfma(a0, pf[nt][0], o[nt][md]);
      o[nt][md] = mfma(a1, pf[nt][1], o[nt][md]);
    }
  }
  // the next page's transposing writes must not pass these reads
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int NT>
__device__ __forceinline__ void attend(const KFrag& k, VFrag& v, int valid, const u32x4 (&qf)[NT][2],
                                       f32x4 (&o)[NT][4], float (&m_run)[NT], float (&l_run)[NT],
                                       float c, unsigned char* vt, int lane) {
  if (valid >= kPage)
    attend_page<NT, false>(k, v, valid, qf, o, m_run, l_run, c, vt, lane);
  else
    attend_page<NT, true>(k, v, valid, qf, o, m_run, l_run, c, vt, lane);
}

__device__ __forceinline__ void flag(int32_t* status, int bit) {
  if (status) atomicOr(status, bit);
}

// One 64-value head row held by 8 lanes (8 values each, lane u has dims 8u..8u+7):
// RMSNorm with weight w, then NeoX rotation with the (cos, sin) row `cs`.
__device__ __forceinline__ void norm_rope_row(float (&x)[8], const uint16_t* w, float eps,
                                              const float2* cs, int u) {
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
  ss += __shfl_xor(ss, 1);
  ss += __shfl_xor(ss, 2);
  ss += __shfl_xor(ss, 4);
  const float inv = 1.0f / sqrtf(ss * (1.0f / kD) + eps);
  const u32x4 wr = ld16(w + 8 * u);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float we = (e & 1) ? bf_hi(wr[e >> 1]) : bf_lo(wr[e >> 1]);
    x[e] = x[e] * inv * we;
  }
  float z[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = __shfl_xor(x[e], 4);
  const float sgn = (u < 4) ? -1.0f : 1.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float2 t = cs[8 * (u & 3) + e];
    x[e] = fmaf(x[e], t.x, sgn * z[e] * t.y);
  }
}

__device__ __forceinline__ void unpack8(u32x4 raw, float (&x)[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    x[2 * q] = bf_lo(raw[q]);
    x[2 * q + 1] = bf_hi(raw[q]);
  }
}

__device__ __forceinline__ u32x4 pack8(const float (&x)[8]) {
  u32x4 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] = pack_bf16x2(x[2 * q], x[2 * q + 1]);
  return r;
}

// ---------------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------------
template <int NT, bool QKNORM, bool POS64>
__global__ __launch_bounds__(kThreads) void drafter_attn_kernel(const Params p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSmemBytes];
  const int s = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = p.T;
  const int nrows = kG * T;
  const int rg = r * p.Hkv + g;

  // ---- a1: lengths (device values, clamped into the contract)
  int L = p.ctx_lens[r];
  const int maxL = p.pt_stride * kPage;
  if (L < 0 || L > maxL) {
    if (tid == 0 && s == 0 && g == 0) flag(p.status, DA_FLAG_CONTEXT_LEN);
    L = L < 0 ? 0 : maxL;
  }
  int b = T;
  if (p.blk_lens) {
    b = p.blk_lens[r];
    if (b < 1 || b > T) {
      if (tid == 0 && s == 0 && g == 0) flag(p.status, DA_FLAG_BLOCK_LEN);
      b = b < 1 ? 1 : T;
    }
  }
  const int npg = (L + kPage - 1) / kPage;
  const int pbeg = s * p.Ps;
  const int pend = min(npg, pbeg + p.Ps);
  const bool own = (s == p.S - 1);

  float2* cs = reinterpret_cast<float2*>(smem + kOffCS);
  // ---- a2/a3 (qknorm): rotation table, one (token, frequency) per thread
  if (QKNORM) {
    if (tid < T * 32) {
      const int t = tid >> 5, i = tid & 31;
      const int64_t pos = POS64 ? static_cast<const int64_t*>(p.positions)[r * T + t]
                                : static_cast<int64_t>(static_cast<const int32_t*>(p.positions)[r * T + t]);
      const double inv_freq = exp2(-static_cast<double>(i) * (1.0 / 32.0) * p.log2_base);  // base^(-2i/64)
      const double th = static_cast<double>(pos) * inv_freq;
      const double kq = rint(th * 0.15915494309189535);          // 1 / (2 pi)
      const double red = fma(-kq, 6.283185307179586, th);        // |red| <= pi (+ tiny)
      float sn, cn;
      sincosf(static_cast<float>(red), &sn, &cn);
      cs[tid] = make_float2(cn, sn);
    }
    __syncthreads();
  }

  // ---- a4: query tile (and own-block K/V tiles) into LDS
  {
    const int sub = tid >> 3, u = tid & 7;
    unsigned char* qt = smem + kOffQ;
    for (int n = sub; n < 16 * NT; n += kThreads / 8) {
      const int t = n / kG;
      float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (n < nrows && t < b) {
        const int h = kG * g + (n - kG * t);
        unpack8(ld16(p.qkv + static_cast<int64_t>(r * T + t) * p.qkv_stride + h * kD + 8 * u), x);
        if (QKNORM) norm_rope_row(x, p.wq, p.eps, cs + t * 32, u);
      }
      *reinterpret_cast<u32x4*>(qt + tile_off(n, u)) = pack8(x);
    }
    if (own) {
      unsigned char* kt = smem + kOffKown;
      unsigned char* vtile = smem + kOffVown;
      for (int item = sub; item < 2 * kPage; item += kThreads / 8) {
        const int j = item & (kPage - 1);
        const bool is_v = item >= kPage;
        float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (j < b) {
          const int col = (is_v ? (p.Hq + p.Hkv + g) : (p.Hq + g)) * kD + 8 * u;
          unpack8(ld16(p.qkv + static_cast<int64_t>(r * T + j) * p.qkv_stride + col), x);
          if (QKNORM && !is_v) norm_rope_row(x, p.wk, p.eps, cs + j * 32, u);
        }
        *reinterpret_cast<u32x4*>((is_v ? vtile : kt) + tile_off(j, u)) = pack8(x);
      }
    }
  }
  __syncthreads();

  // query B-fragments: column (lane & 15) of N-tile nt, dims 32*ks + 8*(lane>>4) ..
  u32x4 qf[NT][2];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      qf[nt][ks] = *reinterpret_cast<const u32x4*>(smem + kOffQ + tile_off(16 * nt + (lane & 15), 4 * ks + (lane >> 4)));

  f32x4 o[NT][4];
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
#pragma unroll
    for (int md = 0; md < 4; ++md) o[nt][md] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  unsigned char* vt = smem + kOffVT + w * kTileBytes;

  // ---- a10: the block's own keys (one 64-slot pseudo-page, b valid), on the least loaded wave
  const int npages_split = max(0, pend - pbeg);
  if (own && w == (npages_split & (kWaves - 1))) {
    KFrag k;
    VFrag v;
    load_k_lds(k, smem + kOffKown, lane);
    load_v_lds(v, smem + kOffVown, lane);
    attend<NT>(k, v, b, qf, o, m_run, l_run, p.c, vt, lane);
  }

  // ---- a5..a9: context pages, next page's loads in flight during the current one
  {
    const int32_t* prow = p.page_table + static_cast<int64_t>(r) * p.pt_stride;
    const int64_t head_off = static_cast<int64_t>(g) * kPage * kD;
    auto page_base = [&](int j, const uint16_t* pool) -> const uint16_t* {
      int phys = prow[j];
      if (phys < 0 || phys >= p.num_pages) {
        flag(p.status, DA_FLAG_PAGE_ID);
        phys = phys < 0 ? 0 : p.num_pages - 1;
      }
      return pool + static_cast<int64_t>(phys) * p.page_stride + head_off;
    };
    int j = pbeg + w;
    KFrag kA, kB;
    VFrag vA, vB;
    if (j < pend) {
      load_k_global(kA, page_base(j, p.kpool), lane);
      load_v_global(vA, page_base(j, p.vpool), lane);
    }
    while (j < pend) {
      int jn = j + kWaves;
      if (jn < pend) {
        load_k_global(kB, page_base(jn, p.kpool), lane);
        load_v_global(vB, page_base(jn, p.vpool), lane);
      }
      attend<NT>(kA, vA, L - j * kPage, qf, o, m_run, l_run, p.c, vt, lane);
      j = jn;
      if (j >= pend) break;
      jn = j + kWaves;
      if (jn < pend) {
        load_k_global(kA, page_base(jn, p.kpool), lane);
        load_v_global(vA, page_base(jn, p.vpool), lane);
      }
      attend<NT>(kB, vB, L - j * kPage, qf, o, m_run, l_run, p.c, vt, lane);
      j = jn;
    }
  }

  // ---- merge the 4 waves (fixed order) into this workgroup's partial
  float* mW = reinterpret_cast<float*>(smem + kOffMW);
  float* lW = reinterpret_cast<float*>(smem + kOffLW);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    l_run[nt] += __shfl_xor(l_run[nt], 16);
    l_run[nt] += __shfl_xor(l_run[nt], 32);
  }
  if (lane < 16) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      mW[w * kRows + 16 * nt + lane] = m_run[nt];
      lW[w * kRows + 16 * nt + lane] = l_run[nt];
    }
  }
  __syncthreads();  // also: every wave is done with its V^T tile and the own-block tiles
  float* obuf = reinterpret_cast<float*>(smem + kOffObuf);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int col = 16 * nt + (lane & 15);
    const float M = fmaxf(fmaxf(mW[col], mW[kRows + col]), fmaxf(mW[2 * kRows + col], mW[3 * kRows + col]));
    const float f = (m_run[nt] == -INFINITY) ? 0.f : fast_exp2((m_run[nt] - M) * p.c);
#pragma unroll
    for (int md = 0; md < 4; ++md) {
      const f32x4 v = o[nt][md] * f;
      *reinterpret_cast<f32x4*>(obuf + (w * kRows + col) * kObufStride + 16 * md + 4 * (lane >> 4)) = v;
    }
  }
  __syncthreads();
  const int rgs = rg * p.S + s;
  {
    float* po = p.part_o + static_cast<int64_t>(rgs) * kRows * kD;
    for (int idx = tid; idx < 16 * NT * (kD / 4); idx += kThreads) {
      const int col = idx >> 4, d4 = (idx & 15) * 4;
      f32x4 acc = *reinterpret_cast<const f32x4*>(obuf + col * kObufStride + d4);
#pragma unroll
      for (int ww = 1; ww < kWaves; ++ww)
        acc += *reinterpret_cast<const f32x4*>(obuf + (ww * kRows + col) * kObufStride + d4);
      *reinterpret_cast<f32x4*>(po + col * kD + d4) = acc;
    }
    if (tid < 16 * NT) {
      const int col = tid;
      float M = mW[col];
#pragma unroll
      for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, mW[ww * kRows + col]);
      float Ls = 0.f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float mw = mW[ww * kRows + col];
        Ls += (mw == -INFINITY) ? 0.f : lW[ww * kRows + col] * fast_exp2((mw - M) * p.c);
      }
      float* pm = p.part_ml + (static_cast<int64_t>(rgs) * kRows + col) * 2;
      pm[0] = M;
      pm[1] = Ls;
    }
  }

  // ---- a11/a12: the last workgroup of (r, g) merges the splits
  __threadfence();
  __syncthreads();
  int* last = reinterpret_cast<int*>(smem + kOffFlag);
  if (tid == 0) {
    const uint32_t prev = atomicAdd(p.counters + rg, 1u);
    const int is_last = (prev == static_cast<uint32_t>(p.S - 1));
    if (is_last) atomicExch(p.counters + rg, 0u);
    *last = is_last;
  }
  __syncthreads();
  if (!*last) return;
  __threadfence();

  float* wts = reinterpret_cast<float*>(smem + kOffWts);
  const int S = p.S;
  if (tid < nrows) {
    const int col = tid;
    const float* ml = p.part_ml + (static_cast<int64_t>(rg) * S * kRows + col) * 2;
    float M = -INFINITY;
    for (int ss = 0; ss < S; ++ss) M = fmaxf(M, ml[ss * kRows * 2]);
    float den = 0.f;
    for (int ss = 0; ss < S; ++ss) {
      const float m = ml[ss * kRows * 2];
      const float e = (m == -INFINITY) ? 0.f : fast_exp2((m - M) * p.c);
      wts[ss * kRows + col] = e;
      den = fmaf(ml[ss * kRows * 2 + 1], e, den);
    }
    const float inv = 1.0f / den;
    for (int ss = 0; ss < S; ++ss) wts[ss * kRows + col] *= inv;
  }
  __syncthreads();
  const float* po = p.part_o + static_cast<int64_t>(rg) * S * kRows * kD;
  for (int idx = tid; idx < nrows * kD; idx += kThreads) {
    const int col = idx >> 6, d = idx & (kD - 1);
    const int t = col / kG, hh = col - kG * t;
    float acc = 0.f;
    if (t < b) {
      for (int ss = 0; ss < S; ++ss)
        acc = fmaf(wts[ss * kRows + col], po[(static_cast<int64_t>(ss) * kRows + col) * kD + d], acc);
    }
    p.out[static_cast<int64_t>(r * T + t) * p.out_stride + (kG * g + hh) * kD + d] = to_bf16(acc);
  }
}

// ---------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

struct Plan {
  int S, Ps;
};

// Split plan from host-known sizes only.  Aim for about one workgroup per
// compute unit over the whole (request, KV head, page) space, with a page count
// per split that is a multiple of the 4 waves once splits hold more than a few
// pages; at most kMaxSplits splits.
Plan make_plan(int R, int Hkv, int stride) {
  constexpr int kTargetWorkgroups = 256;
  if (stride <= 0) return {1, 1};
  const int64_t units = static_cast<int64_t>(R) * Hkv * stride;
  int ps = static_cast<int>((units + kTargetWorkgroups - 1) / kTargetWorkgroups);
  if (ps < 1) ps = 1;
  if (ps > kWaves) ps = (ps + kWaves - 1) / kWaves * kWaves;
  int S = (stride + ps - 1) / ps;
  if (S > kMaxSplits) {
    ps = (stride + kMaxSplits - 1) / kMaxSplits;
    ps = (ps + kWaves - 1) / kWaves * kWaves;
    S = (stride + ps - 1) / ps;
  }
  return {S, ps};
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct WsLayout {
  size_t counters, part_o, part_ml, total;
};

WsLayout ws_layout(int R, int Hkv, int S) {
  WsLayout l;
  l.counters = 0;
  l.part_o = align256(static_cast<size_t>(R) * Hkv * 4);
  l.part_ml = l.part_o + align256(static_cast<size_t>(R) * Hkv * S * kRows * kD * 4);
  l.total = l.part_ml + align256(static_cast<size_t>(R) * Hkv * S * kRows * 2 * 4);
  return l;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Common {
  const void* qkv;
  int64_t qkv_row_stride;
  const void* k_pool;
  const void* v_pool;
  int64_t pool_page_stride;
  int32_t num_pages;
  const int32_t* page_table;
  int32_t page_table_stride;
  const int32_t* context_lens;
  const int32_t* block_lens;
  int32_t R, T, Hq, Hkv, head_dim, page_size;
  float scale;
  void* workspace;
  size_t workspace_bytes;
  void* out;
  int64_t out_row_stride;
  int32_t* status_word;
  void* stream;
};

int check_sizes(int R, int T, int Hq, int Hkv, int head_dim, int page_size, int stride) {
  if (head_dim != kD) return fail(DA_EUNSUPPORTED, "head_dim must be 64");
  if (page_size != kPage) return fail(DA_EUNSUPPORTED, "page_size must be 64");
  if (R < 1 || R > DA_MAX_REQUESTS) return fail(DA_EINVAL, "num_requests must be in [1, 8]");
  if (T < 1 || T > DA_MAX_TOKENS) return fail(DA_EINVAL, "tokens_per_block must be in [1, 8]");
  if (Hkv < 1 || Hkv > DA_MAX_KV_HEADS) return fail(DA_EINVAL, "num_kv_heads must be in [1, 16]");
  if (Hq != kG * Hkv) return fail(DA_EUNSUPPORTED, "num_q_heads must be 6 * num_kv_heads");
  if (stride < 0) return fail(DA_EINVAL, "page_table_stride must be >= 0");
  return DA_OK;
}

int validate(const Common& a, size_t need_ws) {
  int rc = check_sizes(a.R, a.T, a.Hq, a.Hkv, a.head_dim, a.page_size, a.page_table_stride);
  if (rc != DA_OK) return rc;
  if (!a.qkv || !a.out || !a.context_lens) return fail(DA_EINVAL, "qkv, out and context_lens must be non-NULL");
  if (a.page_table_stride > 0) {
    if (!a.page_table) return fail(DA_EINVAL, "page_table must be non-NULL when page_table_stride > 0");
    if (!a.k_pool || !a.v_pool) return fail(DA_EINVAL, "k_pool and v_pool must be non-NULL when page_table_stride > 0");
    if (a.num_pages < 1) return fail(DA_EINVAL, "num_pages must be >= 1 when page_table_stride > 0");
    if (a.pool_page_stride < static_cast<int64_t>(a.Hkv) * kPage * kD)
      return fail(DA_EINVAL, "pool_page_stride must be >= num_kv_heads * 64 * 64");
    if (a.pool_page_stride % 8) return fail(DA_EINVAL, "pool_page_stride must be a multiple of 8 elements");
    if (!aligned16(a.k_pool) || !aligned16(a.v_pool)) return fail(DA_EINVAL, "k_pool and v_pool must be 16-byte aligned");
  }
  const int64_t width = static_cast<int64_t>(a.Hq + 2 * a.Hkv) * kD;
  if (a.qkv_row_stride < width) return fail(DA_EINVAL, "qkv_row_stride must be >= (Hq + 2*Hkv) * 64");
  if (a.qkv_row_stride % 8) return fail(DA_EINVAL, "qkv_row_stride must be a multiple of 8 elements");
  if (a.out_row_stride < static_cast<int64_t>(a.Hq) * kD) return fail(DA_EINVAL, "out_row_stride must be >= Hq * 64");
  if (a.out_row_stride % 8) return fail(DA_EINVAL, "out_row_stride must be a multiple of 8 elements");
  if (!aligned16(a.qkv) || !aligned16(a.out)) return fail(DA_EINVAL, "qkv and out must be 16-byte aligned");
  if (!(std::isfinite(a.scale) && a.scale > 0.f)) return fail(DA_EINVAL, "scale must be finite and > 0");
  if (!a.workspace || a.workspace_bytes < need_ws)
    return fail(DA_EWORKSPACE, "workspace missing or smaller than drafter_attn_workspace_bytes()");
  // aliasing: out must not overlap any input or the workspace; the workspace no input
  const int64_t rows = static_cast<int64_t>(a.R) * a.T;
  const size_t out_n = static_cast<size_t>(((rows - 1) * a.out_row_stride + a.Hq * kD) * 2);
  const size_t qkv_n = static_cast<size_t>(((rows - 1) * a.qkv_row_stride + width) * 2);
  const size_t pool_n = a.page_table_stride > 0
      ? static_cast<size_t>(((static_cast<int64_t>(a.num_pages) - 1) * a.pool_page_stride + static_cast<int64_t>(a.Hkv) * kPage * kD) * 2)
      : 0;
  const size_t pt_n = static_cast<size_t>(a.R) * a.page_table_stride * 4;
  const size_t r_n = static_cast<size_t>(a.R) * 4;
  struct Rng { const void* p; size_t n; const char* name; } ins[] = {
      {a.qkv, qkv_n, "qkv"}, {a.k_pool, pool_n, "k_pool"}, {a.v_pool, pool_n, "v_pool"},
      {a.page_table, pt_n, "page_table"}, {a.context_lens, r_n, "context_lens"},
      {a.block_lens, r_n, "block_lens"}};
  for (const Rng& in : ins) {
    if (overlaps(a.out, out_n, in.p, in.n)) return fail(DA_EINVAL, std::string("out overlaps ") + in.name);
    if (overlaps(a.workspace, need_ws, in.p, in.n)) return fail(DA_EINVAL, std::string("workspace overlaps ") + in.name);
  }
  if (overlaps(a.out, out_n, a.workspace, need_ws)) return fail(DA_EINVAL, "out overlaps workspace");
  if (a.status_word && (overlaps(a.status_word, 4, a.out, out_n) || overlaps(a.status_word, 4, a.workspace, need_ws)))
    return fail(DA_EINVAL, "status_word overlaps out or workspace");
  return DA_OK;
}

Params make_params(const Common& a, const Plan& plan) {
  Params p;
  std::memset(&p, 0, sizeof(p));
  const WsLayout l = ws_layout(a.R, a.Hkv, plan.S);
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  p.qkv = static_cast<const uint16_t*>(a.qkv);
  p.qkv_stride = a.qkv_row_stride;
  p.kpool = static_cast<const uint16_t*>(a.k_pool);
  p.vpool = static_cast<const uint16_t*>(a.v_pool);
  p.page_stride = a.pool_page_stride;
  p.page_table = a.page_table;
  p.ctx_lens = a.context_lens;
  p.blk_lens = a.block_lens;
  p.counters = reinterpret_cast<uint32_t*>(ws + l.counters);
  p.part_o = reinterpret_cast<float*>(ws + l.part_o);
  p.part_ml = reinterpret_cast<float*>(ws + l.part_ml);
  p.out = static_cast<uint16_t*>(a.out);
  p.out_stride = a.out_row_stride;
  p.status = a.status_word;
  p.num_pages = a.num_pages;
  p.pt_stride = a.page_table_stride;
  p.R = a.R;
  p.T = a.T;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.S = plan.S;
  p.Ps = plan.Ps;
  p.c = static_cast<float>(static_cast<double>(a.scale) * 1.4426950408889634);  // log2(e)
  return p;
}

template <int NT, bool QK, bool P64>
int launch_t(const Params& p, const Plan& plan, hipStream_t stream) {
  dim3 grid(plan.S, p.Hkv, p.R);
  hipLaunchKernelGGL((drafter_attn_kernel<NT, QK, P64>), grid, dim3(kThreads), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DA_ELAUNCH, std::string("launch failed: ") + hipGetErrorString(e));
  return DA_OK;
}

template <bool QK, bool P64>
int launch_nt(const Params& p, const Plan& plan, hipStream_t stream) {
  const int nt = (kG * p.T + 15) / 16;
  if (nt == 1) return launch_t<1, QK, P64>(p, plan, stream);
  if (nt == 2) return launch_t<2, QK, P64>(p, plan, stream);
  return launch_t<3, QK, P64>(p, plan, stream);
}

}  // namespace

extern "C" {

size_t drafter_attn_workspace_bytes(int32_t num_requests, int32_t tokens_per_block, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t page_table_stride) {
  if (check_sizes(num_requests, tokens_per_block, num_q_heads, num_kv_heads, kD, kPage, page_table_stride) != DA_OK)
    return 0;
  const Plan plan = make_plan(num_requests, num_kv_heads, page_table_stride);
  return ws_layout(num_requests, num_kv_heads, plan.S).total;
}

int drafter_attn_plan(int32_t num_requests, int32_t num_kv_heads, int32_t page_table_stride,
                      int32_t* num_splits, int32_t* pages_per_split) {
  if (num_requests < 1 || num_requests > DA_MAX_REQUESTS || num_kv_heads < 1 ||
      num_kv_heads > DA_MAX_KV_HEADS || page_table_stride < 0)
    return fail(DA_EINVAL, "plan: sizes outside the contract");
  const Plan plan = make_plan(num_requests, num_kv_heads, page_table_stride);
  if (num_splits) *num_splits = plan.S;
  if (pages_per_split) *pages_per_split = plan.Ps;
  return DA_OK;
}

int drafter_attn(const void* qkv, int64_t qkv_row_stride, const void* k_pool, const void* v_pool,
                 int64_t pool_page_stride, int32_t num_pages, const int32_t* page_table,
                 int32_t page_table_stride, const int32_t* context_lens, const int32_t* block_lens,
                 int32_t num_requests, int32_t tokens_per_block, int32_t num_q_heads, int32_t num_kv_heads,
                 int32_t head_dim, int32_t page_size, float scale, void* workspace, size_t workspace_bytes,
                 void* out, int64_t out_row_stride, int32_t* status_word, void* stream) {
  const Common a{qkv, qkv_row_stride, k_pool, v_pool, pool_page_stride, num_pages, page_table, page_table_stride,
                 context_lens, block_lens, num_requests, tokens_per_block, num_q_heads, num_kv_heads, head_dim,
                 page_size, scale, workspace, workspace_bytes, out, out_row_stride, status_word, stream};
  const size_t need = drafter_attn_workspace_bytes(num_requests, tokens_per_block, num_q_heads, num_kv_heads,
                                                   page_table_stride);
  int rc = validate(a, need);
  if (rc != DA_OK) return rc;
  const Plan plan = make_plan(num_requests, num_kv_heads, page_table_stride);
  Params p = make_params(a, plan);
  g_last_error.clear();
  return launch_nt<false, false>(p, plan, static_cast<hipStream_t>(stream));
}

int drafter_attn_qknorm(const void* qkv, int64_t qkv_row_stride, const void* k_pool, const void* v_pool,
                        int64_t pool_page_stride, int32_t num_pages, const int32_t* page_table,
                        int32_t page_table_stride, const int32_t* context_lens, const int32_t* block_lens,
                        int32_t num_requests, int32_t tokens_per_block, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t page_size, float scale,
                        const void* positions, int32_t positions_dtype, const void* q_norm_weight,
                        const void* k_norm_weight, float eps, float rope_base, void* workspace,
                        size_t workspace_bytes, void* out, int64_t out_row_stride, int32_t* status_word,
                        void* stream) {
  const Common a{qkv, qkv_row_stride, k_pool, v_pool, pool_page_stride, num_pages, page_table, page_table_stride,
                 context_lens, block_lens, num_requests, tokens_per_block, num_q_heads, num_kv_heads, head_dim,
                 page_size, scale, workspace, workspace_bytes, out, out_row_stride, status_word, stream};
  const size_t need = drafter_attn_workspace_bytes(num_requests, tokens_per_block, num_q_heads, num_kv_heads,
                                                   page_table_stride);
  int rc = validate(a, need);
  if (rc != DA_OK) return rc;
  if (!positions || !q_norm_weight || !k_norm_weight)
    return fail(DA_EINVAL, "positions, q_norm_weight and k_norm_weight must be non-NULL");
  if (positions_dtype != DA_POS_INT32 && positions_dtype != DA_POS_INT64)
    return fail(DA_EINVAL, "positions_dtype must be DA_POS_INT32 or DA_POS_INT64");
  if (!(std::isfinite(eps) && eps >= 0.f)) return fail(DA_EINVAL, "eps must be finite and >= 0");
  if (!(std::isfinite(rope_base) && rope_base > 0.f)) return fail(DA_EINVAL, "rope_base must be finite and > 0");
  if (!aligned16(q_norm_weight) || !aligned16(k_norm_weight))
    return fail(DA_EINVAL, "q_norm_weight and k_norm_weight must be 16-byte aligned");
  const int64_t rows = static_cast<int64_t>(num_requests) * tokens_per_block;
  const size_t out_n = static_cast<size_t>(((rows - 1) * out_row_stride + num_q_heads * kD) * 2);
  const size_t pos_n = static_cast<size_t>(rows) * (positions_dtype == DA_POS_INT64 ? 8 : 4);
  if (overlaps(out, out_n, positions, pos_n) || overlaps(out, out_n, q_norm_weight, kD * 2) ||
      overlaps(out, out_n, k_norm_weight, kD * 2))
    return fail(DA_EINVAL, "out overlaps positions or a norm weight");
  if (overlaps(workspace, need, positions, pos_n) || overlaps(workspace, need, q_norm_weight, kD * 2) ||
      overlaps(workspace, need, k_norm_weight, kD * 2))
    return fail(DA_EINVAL, "workspace overlaps positions or a norm weight");
  const Plan plan = make_plan(num_requests, num_kv_heads, page_table_stride);
  Params p = make_params(a, plan);
  p.positions = positions;
  p.wq = static_cast<const uint16_t*>(q_norm_weight);
  p.wk = static_cast<const uint16_t*>(k_norm_weight);
  p.eps = eps;
  p.log2_base = std::log2(static_cast<double>(rope_base));
  g_last_error.clear();
  hipStream_t st = static_cast<hipStream_t>(stream);
  return positions_dtype == DA_POS_INT64 ? launch_nt<true, true>(p, plan, st) : launch_nt<true, false>(p, plan, st);
}

const char* drafter_attn_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
