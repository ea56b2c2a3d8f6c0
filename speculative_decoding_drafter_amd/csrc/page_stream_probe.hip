// Memory-pattern ceiling of the drafter attention's context read (measurement only).
//
// The attention reads, for every (request, KV head), the request's context pages
// through its page-table row: one [64 keys][64 dims] bf16 K tile and one V tile,
// 8 KiB each and contiguous in the HND pool, per page.  This library streams exactly
// those tiles with exactly the attention's launch shape (one 512-thread workgroup per
// (split, KV head, request), the same LDS footprint so one workgroup fits a CU, page
// i of a split on wave i mod 8), and does no arithmetic on them, so that its time is
// what the access pattern itself costs.  Modes:
//   0  LDS DMA with the non-temporal hint, one K slot and one V slot per wave, each
//      refilled as soon as it has landed and been read (the attention's load path)
//   1  the same without the non-temporal hint
//   2  plain 16-byte loads into registers (non-temporal), two pages in flight per wave
//   3  a contiguous read of as many bytes from the start of the K pool (the chip's
//      streaming rate, no page table)
// Every wave folds what it read into one word of `out` (one word per wave), so no read
// can be dropped.  Not part of the attention's interface: bench.py loads it to report
// the attention's time against this ceiling.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 8192;                          // bytes of one K or V tile
constexpr int kSlotBase = 14336;                     // the attention's LDS below its page slots
constexpr int kSmem = kSlotBase + kWaves * 2 * kTile;  // same LDS size: one workgroup per CU
constexpr int kMaxPagesPerSplit = 64 * kWaves;       // a wave's page ids fit one VGPR

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) u32x4 gvec;  // global memory: global_load, not flat

struct Args {
  const uint8_t* k;
  const uint8_t* v;
  int64_t page_bytes;  // bytes from one page to the next (all KV heads)
  int64_t num_pages;
  const int32_t* page_table;
  int32_t pt_stride;
  const int32_t* lens;
  int32_t R, Hkv, S, Ps;
  int64_t stream_vecs;  // mode 3: 16-byte vectors to read from the start of the K pool
  uint32_t* out;
};

__device__ __forceinline__ uint32_t to_lds(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)(p)));
}

__device__ __forceinline__ const uint8_t* in_sgprs(const uint8_t* p) {
  const uint64_t a = reinterpret_cast<uintptr_t>(p);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a))));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a >> 32))));
  return reinterpret_cast<const uint8_t*>(static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32));
}

// One tile (8 KiB) into LDS: 8 DMA instructions of 1 KiB, lane l writing bytes 16l..16l+15
// of each KiB.  m0 holds the LDS base (set here; the compiler does not use m0 in this file).
template <bool NT>
__device__ __forceinline__ void dma_tile(const uint8_t* src, uint32_t lds, uint32_t voff) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint8_t* s = src + 4096 * h;
    if (NT)
      asm volatile(
          "s_mov_b32 m0, %2\n\ts_nop 0\n\t"
          "global_load_lds_dwordx4 %0, %1 nt\n\t"
          "global_load_lds_dwordx4 %0, %1 offset:1024 nt\n\t"
          "global_load_lds_dwordx4 %0, %1 offset:2048 nt\n\t"
          "global_load_lds_dwordx4 %0, %1 offset:3072 nt" ::"v"(voff),
          "s"(s), "s"(lds + 4096 * h)
          : "memory");
    else
      asm volatile(
          "s_mov_b32 m0, %2\n\ts_nop 0\n\t"
          "global_load_lds_dwordx4 %0, %1\n\t"
          "global_load_lds_dwordx4 %0, %1 offset:1024\n\t"
          "global_load_lds_dwordx4 %0, %1 offset:2048\n\t"
          "global_load_lds_dwordx4 %0, %1 offset:3072" ::"v"(voff),
          "s"(s), "s"(lds + 4096 * h)
          : "memory");
  }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

__device__ __forceinline__ uint32_t fold(u32x4 x) { return x.x ^ x.y ^ x.z ^ x.w; }

template <int MODE>
__global__ __launch_bounds__(kThreads) void page_stream_kernel(const Args a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmem];
  const int s = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wg = (r * a.Hkv + g) * a.S + s;
  uint32_t acc = 0;

  if (MODE == 3) {
    gvec* k = (gvec*)(a.k);
    const int64_t n = static_cast<int64_t>(gridDim.x) * gridDim.y * gridDim.z * kThreads;
    for (int64_t i = static_cast<int64_t>(wg) * kThreads + threadIdx.x; i < a.stream_vecs; i += 4 * n) {
      u32x4 x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        x[j] = i + j * n < a.stream_vecs ? __builtin_nontemporal_load(k + i + j * n) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 4; ++j) acc ^= fold(x[j]);
    }
  } else {
    int L = a.lens[r];
    L = L < 0 ? 0 : (L > a.pt_stride * 64 ? a.pt_stride * 64 : L);
    const int npg = (L + 63) / 64;
    const int pbeg = s * a.Ps;
    const int pend = min(npg, pbeg + a.Ps);
    const int first = pbeg + w;
    const int cnt = first < pend ? (pend - first + kWaves - 1) / kWaves : 0;
    int id = 0;
    if (lane < cnt) {
      id = a.page_table[static_cast<int64_t>(r) * a.pt_stride + first + kWaves * lane];
      id = id < 0 ? 0 : (id >= a.num_pages ? static_cast<int>(a.num_pages - 1) : id);
    }
    const int64_t head = static_cast<int64_t>(g) * kTile;
    auto page = [&](const uint8_t* pool, int i) {
      return in_sgprs(pool + static_cast<int64_t>(__builtin_amdgcn_readlane(id, i)) * a.page_bytes + head);
    };
    if (MODE == 0 || MODE == 1) {
      constexpr bool NT = MODE == 0;
      uint8_t* kslot = smem + kSlotBase + w * 2 * kTile;
      uint8_t* vslot = kslot + kTile;
      const uint32_t lk = __builtin_amdgcn_readfirstlane(to_lds(kslot));
      const uint32_t lv = lk + kTile;
      const uint32_t voff = 16u * lane;
      if (cnt > 0) {
        dma_tile<NT>(page(a.k, 0), lk, voff);
        dma_tile<NT>(page(a.v, 0), lv, voff);
      }
      for (int i = 0; i < cnt; ++i) {
        const bool more = i + 1 < cnt;
        wait_vm<8>();  // this page's K landed
        acc ^= fold(*reinterpret_cast<volatile __attribute__((address_space(3))) u32x4*>(
            (__attribute__((address_space(3))) uint8_t*)(kslot) + 16 * lane));
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (more) dma_tile<NT>(page(a.k, i + 1), lk, voff);
        if (more) wait_vm<8>(); else wait_vm<0>();  // this page's V landed
        acc ^= fold(*reinterpret_cast<volatile __attribute__((address_space(3))) u32x4*>(
            (__attribute__((address_space(3))) uint8_t*)(vslot) + 16 * lane));
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (more) dma_tile<NT>(page(a.v, i + 1), lv, voff);
      }
    } else {  // MODE 2: registers, page i+1 requested before page i is folded
      u32x4 b0[16], b1[16];
      auto load = [&](u32x4* dst, int i) {
        gvec* kp = (gvec*)(page(a.k, i));
        gvec* vp = (gvec*)(page(a.v, i));
#pragma unroll
        for (int j = 0; j < 8; ++j) dst[j] = __builtin_nontemporal_load(kp + 64 * j + lane);
#pragma unroll
        for (int j = 0; j < 8; ++j) dst[8 + j] = __builtin_nontemporal_load(vp + 64 * j + lane);
        __builtin_amdgcn_sched_barrier(0);  // all 16 requests out before any fold waits
      };
      auto fold16 = [&](const u32x4* src) {
#pragma unroll
        for (int j = 0; j < 16; ++j) acc ^= fold(src[j]);
      };
      // two buffers taken in turn (no register copies, no load under a branch inside
      // the loop, so the compiler's waits count only the older buffer's loads)
      if (cnt > 0) load(b0, 0);
      int i = 0;
      for (; i + 2 < cnt; i += 2) {
        load(b1, i + 1);
        fold16(b0);
        load(b0, i + 2);
        fold16(b1);
      }
      if (i + 1 < cnt) {
        load(b1, i + 1);
        fold16(b0);
        fold16(b1);
      } else if (cnt > 0) {
        fold16(b0);
      }
    }
  }
  // one word per wave
  acc ^= __shfl_xor(acc, 32);
  acc ^= __shfl_xor(acc, 16);
  acc ^= __shfl_xor(acc, 8);
  acc ^= __shfl_xor(acc, 4);
  acc ^= __shfl_xor(acc, 2);
  acc ^= __shfl_xor(acc, 1);
  if (lane == 0) a.out[static_cast<int64_t>(wg) * kWaves + w] = acc;
}

}  // namespace

extern "C" {

// Stream the context tiles the attention reads (modes 0-2) or as many bytes contiguously
// from the start of the K pool (mode 3), with the attention's grid (Ps pages per split, S
// splits).  k_pool / v_pool: pages of [Hkv][64][64] bf16, page_bytes apart (K and V may
// interleave, as in one [num_pages][2][Hkv][64][64] buffer).  page_table: [R][pt_stride]
// int32; context_lens: [R] int32 (clamped to [0, 64 * pt_stride]); page ids are clamped to
// [0, num_pages).  out: R * Hkv * S * 8 uint32 words.  Returns 0, or -1 when the arguments
// do not fit (nothing launched), or the HIP error of the launch.
int page_stream_probe(int mode, const void* k_pool, const void* v_pool, int64_t num_pages, int64_t page_bytes,
                      int32_t Hkv, const int32_t* page_table, int32_t pt_stride, const int32_t* context_lens,
                      int32_t R, int32_t S, int32_t Ps, int64_t stream_bytes, uint32_t* out, int64_t out_words,
                      hipStream_t stream) {
  if (mode < 0 || mode > 3 || !k_pool || !v_pool || !page_table || !context_lens || !out) return -1;
  if (R < 1 || R > 64 || Hkv < 1 || Hkv > 64 || S < 1 || S > 1024 || Ps < 1 || Ps > kMaxPagesPerSplit) return -1;
  if (pt_stride < 1 || static_cast<int64_t>(S) * Ps < pt_stride || num_pages < 1 || num_pages > (1ll << 31)) return -1;
  if (page_bytes < static_cast<int64_t>(Hkv) * kTile || page_bytes > (1ll << 32) || page_bytes % 16 != 0) return -1;
  if (out_words < static_cast<int64_t>(R) * Hkv * S * kWaves) return -1;
  const int64_t k_extent = (num_pages - 1) * page_bytes + static_cast<int64_t>(Hkv) * kTile;
  if (mode == 3 && (stream_bytes < 16 || stream_bytes % 16 != 0 || stream_bytes > k_extent)) return -1;
  Args a{static_cast<const uint8_t*>(k_pool), static_cast<const uint8_t*>(v_pool), page_bytes, num_pages,
         page_table, pt_stride, context_lens, R, Hkv, S, Ps, stream_bytes / 16, out};
  const dim3 grid(S, Hkv, R);
  switch (mode) {
    case 0: page_stream_kernel<0><<<grid, kThreads, 0, stream>>>(a); break;
    case 1: page_stream_kernel<1><<<grid, kThreads, 0, stream>>>(a); break;
    case 2: page_stream_kernel<2><<<grid, kThreads, 0, stream>>>(a); break;
    default: page_stream_kernel<3><<<grid, kThreads, 0, stream>>>(a); break;
  }
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
