// drafter_attn.hip -- gfx950 (CDNA4) kernels and C ABI for the DFlash drafter's
// block attention (TensorRT-LLM PR #20532, commits adding k3_drafter_attn /
// k3_drafter_attn_qknorm and their contracts).  The ABI is documented in
// include/drafter_attn.h.
//
// One launch per call.  Workgroup (split s, KV head g, request r), 8 waves:
//   1. prologue: the 6*T query rows of group g (and, in split 0, the block's
//      own K/V rows) go to LDS as bf16; in the qknorm variant each row is
//      RMS-normalised and NeoX-rotated in fp32 on the way (angle in fp64).  A
//      request uses only the splits its context reaches (read on the device);
//      the workgroups of the others return at once.
//   2. page loop: wave w walks every 8th page of the split from its w-th (a
//      4-page split gives its pages to waves 4..7).  Per page:
//      the K and V tiles are copied HBM -> LDS by DMA (global_load_lds), S^T =
//      K.Q^T with v_mfma_f32_16x16x32_bf16, online softmax in the exp2 domain,
//      V^T fragments by transposing LDS reads, O^T += V^T.P^T with MFMA.  The
//      next page's DMA is in flight while the current page computes.
//   3. the 8 waves merge (max, sum, output) through LDS and write one fp32
//      partial per workgroup;
//   4. the last workgroup of each (r, g) (device-scope counter, reset by that
//      workgroup) merges the splits in fixed order and writes bf16 output; a
//      request that fits one split writes its output from that split directly,
//      and under a plan of more than 16 splits a request using more than 16
//      merges in two levels (groups of 8 splits, then the groups).
// Where the plan leaves room, the kernel also reads every request's length and
// may take a balanced split schedule (decided on the device from the lengths).
// Nothing depends on device data except through loads, so the same launch is
// valid for any rewritten lengths / page tables / qkv (graph replay), and the
// split plan and every reduction order follow from the sizes and the lengths
// alone (bit-identical reruns).
//
// Also here: the standalone in-place q/k RMSNorm + NeoX rotation (the same
// per-row arithmetic as the attention prologue), and, as a baseline for the
// path the fused op replaces, the append of the block's K/V to the pool and the
// attention kernel with the own-block path compiled out (pooled keys only).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>

#include "drafter_attn.h"

namespace {

constexpr int kD = 64;        // head_dim
constexpr int kPage = 64;     // tokens per page
constexpr int kG = 6;         // query heads per KV head
constexpr int kMaxT = 8;      // tokens per block
constexpr int kRows = 48;     // kG * kMaxT query rows per workgroup
constexpr int kWaves = 8;                    // two per SIMD
static_assert(8 * (kWaves - 2) >= 48, "waves kWaves-2.. hold no query rows (sub = 8w + lane/8)");
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxSplits = 64;
constexpr int kMaxStride = 16384;            // pages per request row (with 64 splits: <= 256 per split)
constexpr int kMaxPagesPerSplit = 64 * kWaves;  // a wave's page ids fit one 64-lane VGPR
constexpr int kMaxReqSplits = 32;             // balanced plan: splits per request (bounds its combine)
constexpr int kTwoLevel = 16;                 // plans with more splits combine a request in two levels
constexpr int kTileBytes = kPage * kD * 2;   // one [64][64] bf16 tile, 8 KiB
constexpr int kStageBytes = 2 * kTileBytes;  // a wave's K slot then V slot
constexpr float kRescaleLog2 = 8.0f;         // lazy-rescale headroom (exp2 units)
// Arrival counters sit 256 bytes apart: the 8 or so workgroups of every (r, g) bump
// theirs at about the same time, and atomics to one line queue behind each other.
constexpr int kCounterStride = 64;           // uint32 units

// LDS layout (bytes)
constexpr int kOffQ = 0;                                   // [48][64] bf16 query tile
constexpr int kOffCS = kOffQ + kRows * kD * 2;             // [8][32] (cos, sin) fp32
constexpr int kOffOwnK = kOffCS + kMaxT * 32 * 8;          // own block's K rows (8 x 128 B)
constexpr int kOffOwnV = kOffOwnK + kMaxT * kD * 2;        // own block's V rows (8 x 128 B)
constexpr int kOffMW = kOffOwnV + kMaxT * kD * 2;          // [48][8] per-wave running max
constexpr int kOffLW = kOffMW + kWaves * kRows * 4;        // [48][8] per-wave weight sum
constexpr int kOffFlag = kOffLW + kWaves * kRows * 4;      // last-workgroup flag
constexpr int kOffStage = 14336;                           // [8 waves][K | V] page slots
constexpr int kObufStride = kD + 4;  // after the loop a wave's slot holds its [48][68] fp32 output (pad: no bank conflicts)
constexpr int kSmemBytes = kOffStage + kWaves * kStageBytes;
static_assert(kOffFlag + 16 <= kOffStage, "LDS layout");
// the own-block tiles are read like full 64-row tiles (rows past the block are
// masked): their 8 KiB read windows must stay inside the allocation
static_assert(kOffOwnV + kTileBytes <= kSmemBytes, "own-block read window");
static_assert(kRows * kObufStride * 4 <= kStageBytes, "a wave's output fits its page slot");
static_assert(kOffMW % 16 == 0 && kOffLW % 16 == 0, "row statistics are read 16 bytes at a time");
static_assert(kSmemBytes <= 160 * 1024, "gfx950 LDS budget");

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Rotary parameters: frequencies base^(-2i/64), optionally rescaled by YaRN (its
// "NTK-by-parts" frequencies and a temperature factor on q and on k).
struct Rope {
  double log2_base;   // log2(rope_base)
  // YaRN's ramp: gamma_i = clamp((x_i - start) * inv_ramp, 0, 1), with x_i the turns of f_i
  // over the original context (ramp in turns) or -i (ramp in the pair index)
  double turn_scale;  // ramp in turns: L / (2 pi), the turns of a unit frequency over L
  double start;       // where gamma leaves 0: alpha (turns), or -hi (pair index)
  double inv_ramp;    // 1 / (beta - alpha), or 1 / (hi - lo), or huge for a step at lo
  double inv_s;       // YaRN: 1 / factor
  float mscale;       // YaRN: the factor on cos and sin
  int32_t yarn;       // 0: plain frequencies, no factor on cos and sin; 1: ramp in turns; 2: in the pair index
};

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
  uint32_t* counters;  // [R*Hkv][kCounterStride]: word 0, and 1..8 for two-level combines
  uint16_t* out;
  int64_t out_stride;
  int32_t* status;
  int32_t num_pages;
  int32_t pt_stride;
  int32_t R, T, Hq, Hkv;
  int32_t S, Ps;
  // Length-aware scheduling: the balanced plan is taken when the requests' pages N > 0
  // satisfy N <= bal_n and their largest page count <= bal_npg (0, 0: never)
  int32_t bal_n, bal_npg;
  float c;    // scale * log2(e): scores live in the exp2 domain
  float eps;
  Rope rope;
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

// two fp32 -> packed bf16 bits, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Byte offset of LDS memory (the 32-bit address LDS instructions and M0 take).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) void*)(p)));
}

// A 64-bit value known to be equal in every lane, moved to SGPRs.  readfirstlane
// works on 32-bit ints: each half is taken back as uint32_t before widening (a
// signed widening would smear bit 31 of the low half over the high half).
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(v))));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(v >> 32))));
  return static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32);
}

// Four 16-byte-per-lane global -> LDS DMAs (global_load_lds_dwordx4).  The
// instruction offset applies to both addresses: DMA j reads sbase + voff_j +
// 1024*j and lands at lds_base + 1024*j + 16*lane.  sbase and lds_base are
// wave-uniform (SGPRs / M0).  Issued from inline asm so that the compiler does
// not treat every later LDS read as dependent on it (it would wait for all DMA in
// flight); the page loop places its own vmcnt waits.  The tiles are read once per
// call, so the loads carry the non-temporal hint (nt): on the 32k-token workload
// with cold caches a call takes 50.1 us with it and 55.0 us without (interleaved
// A/B); with warm caches both take 48 us.  The asm writes m0 without
// declaring it (clang does not accept m0 as a clobber), which is sound only while the
// compiler itself never uses m0 in this file's device code: a CPU test compiles the
// device code to assembly and checks that every m0 reference is this helper's.
__device__ __forceinline__ void dma16x4(uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3, const void* sbase,
                                        uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %5\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %4 nt\n\t"
      "global_load_lds_dwordx4 %1, %4 offset:1024 nt\n\t"
      "global_load_lds_dwordx4 %2, %4 offset:2048 nt\n\t"
      "global_load_lds_dwordx4 %3, %4 offset:3072 nt"
      :: "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(sbase), "s"(lds_base) : "memory");
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Device-scope 8/16-byte global accesses through a buffer resource: cache policy
// sc1 keeps them coherent across the XCDs' L2s, and the compiler tracks their
// completion like any other load.  Offsets past `bytes` are dropped (stores) or
// read as zero (loads) by the hardware's range check.
constexpr int kDeviceCoherent = 16;  // buffer cache-policy operand: sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000 /* 32-bit data format */);
}
__device__ __forceinline__ void st_dev_b128(__amdgpu_buffer_rsrc_t r, int off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kDeviceCoherent);
}
__device__ __forceinline__ void st_dev_b64(__amdgpu_buffer_rsrc_t r, int off, f32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, kDeviceCoherent);
}
__device__ __forceinline__ f32x4 ld_dev_b128(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kDeviceCoherent));
}
__device__ __forceinline__ f32x2 ld_dev_b64(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kDeviceCoherent));
}

// every LDS read this wave issued has returned: its slot may be refilled by DMA
__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// 16-byte-chunk XOR swizzles of the 128-byte rows of a staged [64 keys][64 dims]
// tile.  K: the 8 keys a group of 8 lanes reads for one A-fragment land on 8
// distinct chunk columns.  V: the 4 keys one 16-lane group reads together in a
// transposing read (keys 8j + const, j = 0..3) land on 4 disjoint chunk pairs.
__device__ __forceinline__ int swz_k(int key) { return ((key >> 3) & 3) | ((key & 1) << 2); }
__device__ __forceinline__ int swz_v(int key) { return 2 * (((key >> 3) ^ key) & 3); }
// XOR swizzle of the query tile rows (fragment reads: 8 consecutive rows, one chunk)
__device__ __forceinline__ int swz_q(int row) { return ((row >> 3) ^ row) & 7; }

__device__ __forceinline__ int koff(int key, int chunk) { return key * (kD * 2) + ((chunk ^ swz_k(key)) << 4); }
__device__ __forceinline__ int voff(int key, int chunk) { return key * (kD * 2) + ((chunk ^ swz_v(key)) << 4); }
__device__ __forceinline__ int qoff(int row, int chunk) { return row * (kD * 2) + ((chunk ^ swz_q(row)) << 4); }

// The key a lane's A-fragment row / S^T output register stands for.  The 64
// keys of a page are permuted so that the P^T registers a lane owns after the
// score MFMA are exactly its B-fragment of the PV MFMA.  `mt` = 16-key M-tile,
// `r16` = row inside the tile.
__device__ __forceinline__ int key_of(int mt, int r16) {
  return 32 * (mt & 1) + 8 * (r16 & 3) + 4 * (mt >> 1) + (r16 >> 2);
}

// Per-lane source offsets (bytes inside a tile) for stage_tile: DMA jj writes row
// 8*jj + lane/8, chunk column lane%8; the source chunk is the one the row's swizzle
// maps there.  Only jj % 4 matters, so 4 + 4 registers hold every offset.
struct DmaOffsets {
  uint32_t k[4];
  uint32_t v[4];
};

__device__ __forceinline__ DmaOffsets dma_offsets(int lane) {
  const int r0 = lane >> 3, pc = lane & 7;
  DmaOffsets d;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    d.k[j] = r0 * (kD * 2) + ((pc ^ swz_k(8 * j + r0)) << 4);
    d.v[j] = r0 * (kD * 2) + ((pc ^ swz_v(8 * j + r0)) << 4);
  }
  return d;
}

// Stage one [64][64] bf16 tile (8 KiB contiguous in the pool) into LDS: 8 DMA
// instructions, each reading 1 KiB (8 full rows) of global memory.
template <bool IS_V>
__device__ __forceinline__ void stage_tile(const uint16_t* base, uint32_t lds, const DmaOffsets& off) {
  const uint64_t ua = uniform_u64(reinterpret_cast<uintptr_t>(base));
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const void* sb = reinterpret_cast<const void*>(ua + 4096 * h);
    if (IS_V)
      dma16x4(off.v[0], off.v[1], off.v[2], off.v[3], sb, lds + 4096 * h);
    else
      dma16x4(off.k[0], off.k[1], off.k[2], off.k[3], sb, lds + 4096 * h);
  }
}

struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};

// ---------------------------------------------------------------------------------
// one page (64 keys) of online-softmax attention for one wave, 16*NT query rows,
// from a staged K tile (kt) and V tile (vt)
// ---------------------------------------------------------------------------------
// Hooks let the page loop refill a slot as soon as it has been read:
// k_read() runs once the K tile is in registers, v_wait() before the V tile is
// read, v_read() once the V tile is in registers.
//
// LDS addressing: for the keys a lane reads, both swizzles reduce to a per-lane
// term, so every read is a per-lane base plus a compile-time offset.
//   K: key_of(mt, r16) = 32(mt&1) + 4(mt>>1) + [8(r16&3) + (r16>>2)], and
//      swz_k(key) = (r16&3) | ((r16>>2)&1)<<2 for all mt.
//   V: keys 8e + 4ks + lg all have key&3 = lg, so swz_v(key) = 2*lg.
template <int NT, class KRead = NoHook, class VWait = NoHook, class VRead = NoHook>
__device__ __forceinline__ void attend_page(const unsigned char* kt, const unsigned char* vt, int valid,
                                            const unsigned char* qt, f32x4 (&o)[NT][4],
                                            float (&m_run)[NT], float (&l_run)[NT], float c, int lane,
                                            KRead k_read = {}, VWait v_wait = {}, VRead v_read = {}) {
  const int lg = lane >> 4, r16 = lane & 15;
  const bool tail = valid < kPage;  // wave-uniform
  // query B-fragments (re-read from the LDS tile: fewer live registers across pages)
  u32x4 qf[NT][2];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      qf[nt][ks] = *reinterpret_cast<const u32x4*>(qt + qoff(16 * nt + r16, 4 * ks + lg));
  // ---- K A-fragments: row key_of(mt, r16), dims 32*ks + 8*lg ..
  u32x4 ka[4][2];
  {
    const int sk = (r16 & 3) | (((r16 >> 2) & 1) << 2);
    const unsigned char* kb = kt + (8 * (r16 & 3) + (r16 >> 2)) * (kD * 2);
    const unsigned char* kb0 = kb + ((lg ^ sk) << 4);
    const unsigned char* kb1 = kb + (((4 + lg) ^ sk) << 4);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int row = 32 * (mt & 1) + 4 * (mt >> 1);
      ka[mt][0] = *reinterpret_cast<const u32x4*>(kb0 + row * (kD * 2));
      ka[mt][1] = *reinterpret_cast<const u32x4*>(kb1 + row * (kD * 2));
    }
  }
  // ---- S^T = K . Q^T  (rows: keys, cols: query rows)
  f32x4 s[NT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma(ka[mt][0], qf[nt][0], acc);
      acc = mfma(ka[mt][1], qf[nt][1], acc);
      s[nt][mt] = acc;
    }
  k_read();
  if (tail) {
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
  // ---- V^T A-fragments: row d = 16*md + r16; keys 8e + 4ks + lg, e = 0..7.
  // ds_read_b64_tr_b16 transposes inside each 16-lane group: destination lane
  // 4a + c gets element c of the 8 bytes addressed by lanes 4j + a (j = 0..3).  So
  // lane 4j + a points at V[key_j][16 md + 4a .. +3] with key_j = 8(j + 4h) + 4ks
  // + lg, and every lane receives the 4 keys of its own dimension d.
  v_wait();
  u32x4 va[4][2];
  {
    const int j = r16 >> 2, a = r16 & 3;
    const int t = j ^ lg;  // swz_v(key_j) / 2 for every key this lane addresses
    const unsigned char* vrow = vt + (8 * j + lg) * (kD * 2) + 8 * (a & 1);
#pragma unroll
    for (int md = 0; md < 4; ++md) {
      const unsigned char* vm = vrow + (((2 * md + (a >> 1)) ^ (2 * t)) << 4);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(vm + (32 * h + 4 * ks) * (kD * 2)));
          const uint64_t bits = __builtin_bit_cast(uint64_t, x);
          va[md][ks][2 * h] = static_cast<uint32_t>(bits);
          va[md][ks][2 * h + 1] = static_cast<uint32_t>(bits >> 32);
        }
    }
  }
  v_read();
  if (tail) {
    // slots past the length may hold anything (NaN): zero their values
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k0 = 16 * q + 4 * ks + lg;  // element e = 2q (low half); e = 2q + 1 is k0 + 8
        const uint32_t m = (k0 < valid ? 0x0000ffffu : 0u) | (k0 + 8 < valid ? 0xffff0000u : 0u);
#pragma unroll
        for (int md = 0; md < 4; ++md) va[md][ks][q] &= m;
      }
  }
  // ---- per query N-tile: online softmax (exp2 domain), then O^T += V^T . P^T.
  // The reference maximum m_run only moves when this page's maximum exceeds it by
  // more than kRescaleLog2 (in exp2 units): until then the weights may grow up to
  // 2^kRescaleLog2 (harmless in fp32 and bf16), and the rescale of O and l is
  // skipped when no lane of the wave needs it.
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float mx = s[nt][0][0];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[nt][mt][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (__builtin_amdgcn_ballot_w64((mx - m_run[nt]) * c > kRescaleLog2) != 0) {
      const float m_new = fmaxf(m_run[nt], mx);
      const float alpha = fast_exp2((m_run[nt] - m_new) * c);  // 1 where m_run stays
      m_run[nt] = m_new;
      l_run[nt] *= alpha;
#pragma unroll
      for (int md = 0; md < 4; ++md) o[nt][md] *= alpha;
    }
    const float nmc = -m_run[nt] * c;
    float pr[4][4];
    float lsum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[mt][i] = fast_exp2(fmaf(s[nt][mt][i], c, nmc));
        lsum += pr[mt][i];
      }
    l_run[nt] += lsum;
    u32x4 pf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      pf[ks][0] = pack_bf16x2(pr[2 * ks][0], pr[2 * ks][1]);
      pf[ks][1] = pack_bf16x2(pr[2 * ks][2], pr[2 * ks][3]);
      pf[ks][2] = pack_bf16x2(pr[2 * ks + 1][0], pr[2 * ks + 1][1]);
      pf[ks][3] = pack_bf16x2(pr[2 * ks + 1][2], pr[2 * ks + 1][3]);
    }
#pragma unroll
    for (int md = 0; md < 4; ++md) {
      o[nt][md] = mfma(va[md][0], pf[0], o[nt][md]);
      o[nt][md] = mfma(va[md][1], pf[1], o[nt][md]);
    }
  }
}

// Phase timestamps for measurement builds (DA_PHASE_TRACE defined; the product build
// compiles them out): 64 u64 slots per workgroup, at (uint64_t*)status_word + 64 * the
// workgroup's linear index, each a reading of the 100 MHz real-time counter:
//   [w] wave w starts, [8+w] its prologue loads have landed, [16+w] its share of the
//   prologue is done and its first page's DMA issued, [24+w] that page's K tile has
//   landed, [32+w] its page loop ends, [40] XCC id, [41] after the merge barrier, [42]
//   merged, [43] partial published, [44] counter taken, [45] the combine's loads have
//   landed (with more than 8 splits: every chunk merged), [46] output stored, [47] after the prologue
//   barrier, [48+w] a wave that issues its first page before the prologue has issued it.
//   The status flags are off in such builds.
#ifdef DA_PHASE_TRACE
#define DA_STAMP(slot, cond)                                                              \
  do {                                                                                   \
    const uint64_t da_t = __builtin_amdgcn_s_memrealtime();                             \
    if (cond) da_trace[slot] = da_t;                                                      \
  } while (0)
#define DA_TRACE_BASE(p)                                                                  \
  uint64_t* da_trace = reinterpret_cast<uint64_t*>((p).status) +                          \
                       64 * (blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z))
#else
#define DA_STAMP(slot, cond) \
  do {                       \
  } while (0)
#define DA_TRACE_BASE(p) \
  do {                   \
  } while (0)
#endif

__device__ __forceinline__ void flag(int32_t* status, int bit) {
#ifndef DA_PHASE_TRACE
  if (status) atomicOr(status, bit);
#endif
}

// (cos, sin) of the NeoX angle pos * f_i for frequency i < 32, f_i = base^(-2i/64):
// the angle is formed and reduced modulo 2 pi in fp64 (absolute error about
// |angle| * 2^-52, 2e-6 rad at positions near 2^33, where fp32 could not even hold
// the position), then evaluated in fp32.  With YaRN, f_i is first moved towards
// f_i / s: f_i <- (1 - gamma) f_i / s + gamma f_i, with gamma ramping from 0 to 1
// linearly in the turns f_i makes over the original context or in the pair index
// (the ramp's constants come from the host), and cos and sin carry the factor on q
// and k.
__device__ __forceinline__ float2 rope_cos_sin(int64_t pos, int i, const Rope& rp) {
  double inv_freq = exp2(-static_cast<double>(i) * (1.0 / 32.0) * rp.log2_base);  // base^(-2i/64)
  if (rp.yarn) {
    const double x = rp.yarn == 2 ? -static_cast<double>(i) : rp.turn_scale * inv_freq;
    const double g = fmin(fmax((x - rp.start) * rp.inv_ramp, 0.0), 1.0);
    inv_freq = (1.0 - g) * inv_freq * rp.inv_s + g * inv_freq;
  }
  const double th = static_cast<double>(pos) * inv_freq;
  const double kq = rint(th * 0.15915494309189535);    // 1 / (2 pi)
  const double red = fma(-kq, 6.283185307179586, th);  // |red| <= pi (+ tiny)
  float sn, cn;
  sincosf(static_cast<float>(red), &sn, &cn);
  if (rp.yarn) {
    sn *= rp.mscale;
    cn *= rp.mscale;
  }
  return make_float2(cn, sn);
}

// One 64-value head row held by 8 lanes (8 values each, lane u has dims 8u..8u+7):
// RMSNorm with the weights' 8 bf16 values `wr` for those dims, then NeoX rotation
// with the (cos, sin) row `cs`.
__device__ __forceinline__ void norm_rope_row(float (&x)[8], u32x4 wr, float eps, const float2* cs, int u) {
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
  ss += __shfl_xor(ss, 1);
  ss += __shfl_xor(ss, 2);
  ss += __shfl_xor(ss, 4);
  const float inv = 1.0f / sqrtf(ss * (1.0f / kD) + eps);
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

// x[0..3] -> dims d..d+3 of an output row, x[4..7] -> dims d+32..d+35 (bf16)
__device__ __forceinline__ void store_out8(uint16_t* dst, const float (&x)[8]) {
  *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
  *reinterpret_cast<u32x2*>(dst + 32) = u32x2{pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
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
// OWN = false is the attention of the path the fused op replaces: the block's
// queries attend to pooled keys only (the caller appended the block to the pool and
// passes kv lengths L + b), nothing is read from qkv but the queries.
template <int NT, bool QKNORM, bool POS64, bool OWN = true, bool BAL = false, bool MANY = false>
__global__ __launch_bounds__(kThreads) void drafter_attn_kernel(const Params p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kSmemBytes];
  int s = blockIdx.x, r = blockIdx.z;
  const int g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = p.T;
  const int nrows = kG * T;
  DA_TRACE_BASE(p);
  DA_STAMP(w, lane == 0);

  // ---- a1: every global load of the prologue is issued first and consumed before
  // the first page's DMA: the waits the compiler places before a use cannot tell
  // those loads from the DMA (issued from inline asm), so a load still pending
  // after it would wait for the whole page.
  //
  // The page ids of this wave's pages of the split (every 8th page from `first` --
  // at most 64, so one VGPR holds them and the page loop reads them with readlane,
  // with no memory access of its own) are loaded for the whole split range of the
  // row before the length is known; only the first cnt are used, checked and
  // clamped.
  //
  // A split narrower than the waves (4 pages) gives its pages to the highest
  // waves, which have the least prologue work and issue their first page early.
  int pbeg = s * p.Ps;
  int wshift = p.Ps < kWaves ? kWaves - p.Ps : 0;
  int first = pbeg + w - wshift;
  const int row_end = min(pbeg + p.Ps, p.pt_stride);
  const int cand = (w >= wshift && first < row_end) ? (row_end - first + kWaves - 1) / kWaves : 0;
  int id = 0;
  if (lane < cand) id = p.page_table[static_cast<int64_t>(r) * p.pt_stride + first + kWaves * lane];
  bool own = OWN && s == 0;
  // Thread (sub, u) holds dims 8u .. 8u+7 of one head row: query row sub = 6t + h
  // of the tile (sub < 6T), or, in split 0, row j < T of the block's own K
  // (sub = 48 + j) or V (sub = 56 + j).  Rows past the block length are loaded
  // (they exist) and zeroed below.
  const int sub = tid >> 3, u = tid & 7;
  const int q_t = sub / kG;
  const int oj = (sub - 48) & (kMaxT - 1);
  const bool is_q = sub < nrows;
  const bool own_v = sub >= 48 + kMaxT;
  bool is_own = own && sub >= 48 && sub < 48 + 2 * kMaxT && oj < T;
  u32x4 raw = {0u, 0u, 0u, 0u}, wraw = {0u, 0u, 0u, 0u};
  if (is_q) {
    raw = ld16(p.qkv + static_cast<int64_t>(r * T + q_t) * p.qkv_stride + (kG * g + sub - kG * q_t) * kD + 8 * u);
    if (QKNORM) wraw = ld16(p.wq + 8 * u);
  } else if (is_own) {
    raw = ld16(p.qkv + static_cast<int64_t>(r * T + oj) * p.qkv_stride + (own_v ? p.Hq + p.Hkv + g : p.Hq + g) * kD +
               8 * u);
    if (QKNORM && !own_v) wraw = ld16(p.wk + 8 * u);
  }
  int64_t pos = 0;
  if (QKNORM && tid < T * 32) {
    const int t = tid >> 5;
    pos = POS64 ? static_cast<const int64_t*>(p.positions)[r * T + t]
                : static_cast<int64_t>(static_cast<const int32_t*>(p.positions)[r * T + t]);
  }
  int L = p.ctx_lens[r];
  int b = p.blk_lens ? p.blk_lens[r] : T;
  // With the length-aware schedule compiled in, every request's length is loaded too,
  // by scalar loads: they are only waited for after the first page's DMA (a vector load
  // here would have to land before that DMA is issued).
  int lens[DA_MAX_REQUESTS];
#pragma unroll
  for (int i = 0; i < DA_MAX_REQUESTS; ++i) lens[i] = (BAL && i < p.R) ? p.ctx_lens[i] : 0;
  asm volatile("" ::"v"(raw), "v"(wraw), "v"(pos), "v"(L), "v"(b));  // every prologue load has landed
  DA_STAMP(8 + w, lane == 0);

  const int maxL = p.pt_stride * kPage;
  int L_in = L, b_in = b;  // as loaded, for the status flags
  L = L < 0 ? 0 : (L > maxL ? maxL : L);
  b = b < 1 ? 1 : (b > T ? T : b);
  int npg = (L + kPage - 1) / kPage;
  // A request uses only the splits its pages reach (at least split 0, which holds the
  // block's own keys); its other workgroups have nothing to do (unless the balanced
  // plan below gives them work).  A request that fits one split is answered by that
  // split directly.
  int ps = p.Ps;
  int s_used = max(1, (npg + ps - 1) / ps);
  int slot0 = (r * p.Hkv + g) * p.S;  // the first partial slot of (r, g)
  int pend = min(npg, pbeg + ps);
  // the block's own keys go to a wave with the fewest pages of this split
  int own_wave = (max(0, pend - pbeg) + wshift) & (kWaves - 1);
  int cnt = (w >= wshift && first < pend) ? (pend - first + kWaves - 1) / kWaves : 0;
  if (lane < cnt && (id < 0 || id >= p.num_pages)) {
    flag(p.status, DA_FLAG_PAGE_ID);
    id = id < 0 ? 0 : p.num_pages - 1;
  }
  const int64_t head_off = static_cast<int64_t>(g) * kPage * kD;
  unsigned char* kslot = smem + kOffStage + w * kStageBytes;
  unsigned char* vslot = kslot + kTileBytes;
  const uint32_t lds_k = __builtin_amdgcn_readfirstlane(lds_addr(kslot));
  const uint32_t lds_v = lds_k + kTileBytes;
  auto page_off = [&](int i) {
    return static_cast<int64_t>(__builtin_amdgcn_readlane(id, i)) * p.page_stride + head_off;
  };
  const DmaOffsets doff = dma_offsets(lane);
  // which waves issue their first page before their share of the prologue (see below)
  const bool early_dma = w >= kWaves - 4;
  if (early_dma && cnt > 0) {
    stage_tile<false>(p.kpool + page_off(0), lds_k, doff);
    stage_tile<true>(p.vpool + page_off(0), lds_v, doff);
  }
  DA_STAMP(48 + w, lane == 0 && early_dma && cnt > 0);

  // ---- length-aware split scheduling (BAL), decided while the first pages are in
  // flight.  Every workgroup derives the same schedule from the lengths (device data)
  // and the host sizes, so the same inputs always take the same path and the same
  // reduction order (bit-identical reruns and replays).  Static plan (above):
  // workgroup (x, g, z) takes split x of request z, splits of Ps pages.  Balanced
  // plan: the N pages of all requests are cut into about R*(S-1) splits of Pb pages
  // (a multiple of 8, at least ceil(max npg / kMaxReqSplits)); request i takes
  // max(1, ceil(npg_i / Pb)) consecutive entries, at most R*S in all, and workgroup
  // (x, g, z) takes entry x + S*z of KV head g.  The balanced plan is taken only when
  // it puts at most 3/4 of the pages on a workgroup (Pb <= 3 Ps / 4), i.e. when long
  // requests would otherwise leave many workgroups idle.  It then costs one more round
  // trip: the
  // workgroup loads its balanced split's page ids and rows, and the static split's
  // first page, already in flight, is drained and dropped.
  bool balanced = false;
  if (BAL) {
    int N = 0, npg_max = 0;
#pragma unroll
    for (int i = 0; i < DA_MAX_REQUESTS; ++i) {
      const int n = ((lens[i] < 0 ? 0 : (lens[i] > maxL ? maxL : lens[i])) + kPage - 1) / kPage;
      N += n;
      npg_max = max(npg_max, n);
    }
    // Pb <= 3 Ps / 4 exactly when both bounds hold (thresholds from the host)
    if (__builtin_expect(N > 0 && N <= p.bal_n && npg_max <= p.bal_npg, 0)) {
      balanced = true;
      // lane i < R: request i's length and page count
      int Li = 0;
#pragma unroll
      for (int i = 0; i < DA_MAX_REQUESTS; ++i) Li = lane == i ? lens[i] : Li;
      const int npg_l = ((Li < 0 ? 0 : (Li > maxL ? maxL : Li)) + kPage - 1) / kPage;
      const int X = p.R * (p.S - 1);
      const int pb = max((N + X - 1) / X, (npg_max + kMaxReqSplits - 1) / kMaxReqSplits);
      ps = max(kWaves, (pb + kWaves - 1) / kWaves * kWaves);
      const int k_l = lane < p.R ? max(1, (npg_l + ps - 1) / ps) : 0;
      const int e = blockIdx.x + p.S * blockIdx.z;
      int base = 0, rr = -1;
#pragma nounroll
      for (int i = 0; i < p.R; ++i) {
        const int k = __builtin_amdgcn_readlane(k_l, i);
        if (rr < 0 && e < base + k) {
          rr = i;
          s = e - base;
          s_used = k;
          slot0 = g * p.R * p.S + base;
        }
        base += k;
      }
      if (rr < 0) {  // past the schedule's last entry
        wait_vmcnt<0>();
        return;
      }
      r = rr;
      L_in = __builtin_amdgcn_readlane(Li, r);
      L = L_in < 0 ? 0 : (L_in > maxL ? maxL : L_in);
      npg = __builtin_amdgcn_readlane(npg_l, r);
      pbeg = s * ps;
      wshift = 0;
      first = pbeg + w;
      pend = min(npg, pbeg + ps);
      own_wave = (pend - pbeg) & (kWaves - 1);
      cnt = first < pend ? (pend - first + kWaves - 1) / kWaves : 0;
      own = OWN && s == 0;
      is_own = own && sub >= 48 && sub < 48 + 2 * kMaxT && oj < T;
      id = 0;
      if (lane < cnt) id = p.page_table[static_cast<int64_t>(r) * p.pt_stride + first + kWaves * lane];
      raw = wraw = u32x4{0u, 0u, 0u, 0u};
      if (is_q) {
        raw = ld16(p.qkv + static_cast<int64_t>(r * T + q_t) * p.qkv_stride + (kG * g + sub - kG * q_t) * kD + 8 * u);
        if (QKNORM) wraw = ld16(p.wq + 8 * u);
      } else if (is_own) {
        raw = ld16(p.qkv + static_cast<int64_t>(r * T + oj) * p.qkv_stride +
                   (own_v ? p.Hq + p.Hkv + g : p.Hq + g) * kD + 8 * u);
        if (QKNORM && !own_v) wraw = ld16(p.wk + 8 * u);
      }
      if (QKNORM && tid < T * 32) {
        const int t = tid >> 5;
        pos = POS64 ? static_cast<const int64_t*>(p.positions)[r * T + t]
                    : static_cast<int64_t>(static_cast<const int32_t*>(p.positions)[r * T + t]);
      }
      b = p.blk_lens ? p.blk_lens[r] : T;
      wait_vmcnt<0>();  // these loads, and the static split's first page (its slot is reused)
      asm volatile("" ::"v"(raw), "v"(wraw), "v"(pos), "v"(b), "v"(id));
      b_in = b;
      b = b < 1 ? 1 : (b > T ? T : b);
      if (lane < cnt && (id < 0 || id >= p.num_pages)) {
        flag(p.status, DA_FLAG_PAGE_ID);
        id = id < 0 ? 0 : p.num_pages - 1;
      }
      if (early_dma && cnt > 0) {
        stage_tile<false>(p.kpool + page_off(0), lds_k, doff);
        stage_tile<true>(p.vpool + page_off(0), lds_v, doff);
      }
    }
  }
  if (!balanced && s >= s_used) return;
  const int rg = r * p.Hkv + g;
  if (tid == 0 && s == 0 && g == 0) {  // request r's first split reports its length and block length
    if (L_in < 0 || L_in > maxL) flag(p.status, DA_FLAG_CONTEXT_LEN);
    if (b_in < 1 || b_in > T) flag(p.status, DA_FLAG_BLOCK_LEN);
  }

  float2* cs = reinterpret_cast<float2*>(smem + kOffCS);
  // ---- a2/a3 (qknorm): rotation table, one (token, frequency) per thread
  if (QKNORM) {
    if (tid < T * 32) cs[tid] = rope_cos_sin(pos, tid & 31, p.rope);
    __syncthreads();
  }

  // ---- a4: query tile (and the own block's K/V rows) into LDS as bf16; rows of
  // the tile past 6T and rows past the block length are zero
  if (sub < 16 * NT || is_own) {
    float x[8];
    unpack8(raw, x);
    const int t = is_q ? q_t : oj;
    const bool live = (is_q || is_own) && t < b;
    if (QKNORM && live && !own_v) norm_rope_row(x, wraw, p.eps, cs + t * 32, u);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = live ? x[e] : 0.f;
    unsigned char* dst = sub < 48 ? smem + kOffQ + qoff(sub, u)
                                  : (own_v ? smem + kOffOwnV + voff(oj, u) : smem + kOffOwnK + koff(oj, u));
    *reinterpret_cast<u32x4*>(dst) = pack8(x);
  }
  if (own && sub >= 48 && sub < 48 + 2 * kMaxT && oj >= T) {
    // own-block rows T .. 7 are never valid keys: zero
    *reinterpret_cast<u32x4*>(own_v ? smem + kOffOwnV + voff(oj, u) : smem + kOffOwnK + koff(oj, u)) =
        u32x4{0u, 0u, 0u, 0u};
  }
  // The other waves issue their first page's DMA once their share of the prologue
  // is done (the slots are not touched by the prologue).  A CU takes only about two
  // waves' worth of these 1 KiB DMAs at once; a wave issuing more waits until the
  // memory system drains, so a wave that issued before its prologue work would hold
  // the prologue back.  Waves 4 to 7 (the last 16 query rows and the own block's
  // rows) issue theirs before the prologue: the stream starts early, and the other
  // waves' first pages are still in flight when the page loop starts and requests
  // the second ones.  (Waves 6-7 alone, for splits of more than 16 pages, were
  // 0.3 us slower on 32k-token contexts; all eight waves early, 0.4 us slower.)
  if (!early_dma && cnt > 0) {
    stage_tile<false>(p.kpool + page_off(0), lds_k, doff);
    stage_tile<true>(p.vpool + page_off(0), lds_v, doff);
  }
  DA_STAMP(16 + w, lane == 0);
  __syncthreads();  // the query tile, rotation table and own-block rows are in LDS
  DA_STAMP(47, tid == 0);

  const unsigned char* qt = smem + kOffQ;
  f32x4 o[NT][4];
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
#pragma unroll
    for (int md = 0; md < 4; ++md) o[nt][md] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- a10: the block's own keys (a 64-slot pseudo-page with b valid keys)
  if (own && w == own_wave)
    attend_page<NT>(smem + kOffOwnK, smem + kOffOwnV, b, qt, o, m_run, l_run, p.c, lane);

  // ---- a5..a9: context pages.  One K slot and one V slot per wave, each refilled
  // with the next page as soon as it has been read, so the next page's DMA runs
  // under the rest of this page's work (and the other wave on the SIMD).  Only the
  // request's last page can be partial; if this wave owns it, it is its last one.
  {
    const bool tail = cnt > 0 && first + kWaves * (cnt - 1) == npg - 1 && (L & (kPage - 1)) != 0;
    for (int i = 0; i < cnt; ++i) {
      const bool more = i + 1 < cnt;
      wait_vmcnt<8>();  // this page's K landed (its V may still be in flight)
      DA_STAMP(24 + w, lane == 0 && i == 0);
      auto k_read = [&]() {
        if (more) {
          wait_lds_reads();
          stage_tile<false>(p.kpool + page_off(i + 1), lds_k, doff);
        }
      };
      auto v_wait = [&]() {
        if (more) wait_vmcnt<8>(); else wait_vmcnt<0>();
      };
      auto v_read = [&]() {
        if (more) {
          wait_lds_reads();
          stage_tile<true>(p.vpool + page_off(i + 1), lds_v, doff);
        }
      };
      const int valid = (tail && i == cnt - 1) ? L - (npg - 1) * kPage : kPage;
      attend_page<NT>(kslot, vslot, valid, qt, o, m_run, l_run, p.c, lane, k_read, v_wait, v_read);
    }
  }

  DA_STAMP(32 + w, lane == 0);
#ifdef DA_PHASE_TRACE
  if (tid == 0) da_trace[40] = __builtin_amdgcn_s_getreg(0xF814) & 0xF;  // XCC id
#endif
  // ---- merge the waves (fixed order).  Each wave leaves its running maxima and
  // sums and its unnormalised output in LDS -- the output inside its own page
  // slot, which it no longer reads -- and after one barrier each thread owns one
  // (query row, 8 dims) of the workgroup's merged state.
  float* mW = reinterpret_cast<float*>(smem + kOffMW);  // [48 rows][8 waves]
  float* lW = reinterpret_cast<float*>(smem + kOffLW);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    l_run[nt] += __shfl_xor(l_run[nt], 16);
    l_run[nt] += __shfl_xor(l_run[nt], 32);
  }
  if (lane < 16) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      mW[(16 * nt + lane) * kWaves + w] = m_run[nt];
      lW[(16 * nt + lane) * kWaves + w] = l_run[nt];
    }
  }
  {
    float* ob = reinterpret_cast<float*>(kslot);  // [48][kObufStride] fp32
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int md = 0; md < 4; ++md)
        *reinterpret_cast<f32x4*>(ob + (16 * nt + (lane & 15)) * kObufStride + 16 * md + 4 * (lane >> 4)) =
            o[nt][md];
  }
  __syncthreads();
  DA_STAMP(41, tid == 0);

  // query row (6t + h) and dims 4*oc .. 4*oc+3 and 32+4*oc .. 32+4*oc+3: each
  // 16-byte access of a wave's 8 threads of a row then covers one whole 128-byte
  // line of the row (whole-line writes through the L2)
  const int row = tid >> 3, oc = tid & 7;
  const bool row_thread = row < nrows;
  float acc[8];
  float m_wg = -INFINITY, l_wg = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  if (row_thread) {
    const f32x4 m0 = *reinterpret_cast<const f32x4*>(mW + row * kWaves);
    const f32x4 m1 = *reinterpret_cast<const f32x4*>(mW + row * kWaves + 4);
    const f32x4 l0 = *reinterpret_cast<const f32x4*>(lW + row * kWaves);
    const f32x4 l1 = *reinterpret_cast<const f32x4*>(lW + row * kWaves + 4);
    const float mw[kWaves] = {m0[0], m0[1], m0[2], m0[3], m1[0], m1[1], m1[2], m1[3]};
    const float lw[kWaves] = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) m_wg = fmaxf(m_wg, mw[ww]);
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      // a wave that saw no key has m = -inf, l = 0, o = 0: weight 0
      const float e = (mw[ww] == -INFINITY) ? 0.f : fast_exp2((mw[ww] - m_wg) * p.c);
      l_wg = fmaf(lw[ww], e, l_wg);
      const float* src = reinterpret_cast<const float*>(smem + kOffStage + ww * kStageBytes) +
                         row * kObufStride + 4 * oc;
      const f32x4 a = *reinterpret_cast<const f32x4*>(src);
      const f32x4 c4 = *reinterpret_cast<const f32x4*>(src + 32);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[j] = fmaf(e, a[j], acc[j]);
        acc[4 + j] = fmaf(e, c4[j], acc[4 + j]);
      }
    }
  }
  const int t_row = row / kG;
  uint16_t* out_row = p.out + static_cast<int64_t>(r * T + t_row) * p.out_stride + (kG * g + row - kG * t_row) * kD +
                      4 * oc;
  DA_STAMP(42, tid == 0);
  if (s_used == 1) {
    // a single split: its merged state is the answer (l_wg > 0 unless there is no
    // key at all, possible only without the block's own keys: zero rows then)
    if (row_thread) {
      const float inv = l_wg > 0.f ? 1.0f / l_wg : 0.f;
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = (t_row < b) ? acc[j] * inv : 0.f;
      store_out8(out_row, x);
    }
    DA_STAMP(46, tid == 0);
    return;
  }
  // The partial is published with device-scope stores (coherent across the
  // XCDs' L2s without a cache write-back), completed before the counter
  // increment; the last workgroup reads it back with device-scope loads.
  const int rgs = slot0 + s;
  if (row_thread) {
    const __amdgpu_buffer_rsrc_t po = dev_rsrc(p.part_o + static_cast<int64_t>(rgs) * kRows * kD, kRows * kD * 4);
    const int off = (row * kD + 4 * oc) * 4;
    st_dev_b128(po, off, f32x4{acc[0], acc[1], acc[2], acc[3]});
    st_dev_b128(po, off + 128, f32x4{acc[4], acc[5], acc[6], acc[7]});
    if (oc == 0) {
      const __amdgpu_buffer_rsrc_t pm = dev_rsrc(p.part_ml + static_cast<int64_t>(rgs) * kRows * 2, kRows * 2 * 4);
      st_dev_b64(pm, row * 8, f32x2{m_wg, l_wg});
    }
  }

  // ---- a11/a12: the last workgroup of (r, g) merges the splits
  wait_vmcnt<0>();  // this thread's partial stores are complete (visible at device scope)
  __syncthreads();
  DA_STAMP(43, tid == 0);
  if constexpr (MANY) {
    // A request with more than kTwoLevel splits (plans of more than kTwoLevel splits
    // only: the kernel of the other plans is compiled without this) merges in two
    // levels: the last workgroup of each group of 8 consecutive splits merges its group
    // into the group's first slot (whose partial it has just read back) and publishes
    // it, and the last of the groups merges the groups, in group order -- the partials'
    // loads spread over several CUs instead of one CU reading them all, chunk by chunk.
    if (s_used > kTwoLevel) {
      const int grp = s >> 3;
      const int ngrp = (s_used + 7) >> 3;
      uint32_t* ctr = p.counters + kCounterStride * rg;
      int* flag2 = reinterpret_cast<int*>(smem + kOffFlag);
      if (tid == 0) {
        const int n = min(8, s_used - 8 * grp);
        const uint32_t prev = __hip_atomic_fetch_add(ctr + 1 + grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int is_last = (prev == static_cast<uint32_t>(n - 1));
        if (is_last) __hip_atomic_store(ctr + 1 + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag2 = is_last;
      }
      __syncthreads();
      DA_STAMP(44, tid == 0);
      if (!*flag2) return;
      float sum[8], den2 = 0.f;
      // n <= 8 partials at slots base + stride * j into (maximum, den2, sum)
      auto merge8 = [&](int base, int stride, int n) {
        den2 = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) sum[j] = 0.f;
        const int extent = (n - 1) * stride + 1;
        const __amdgpu_buffer_rsrc_t pm =
            dev_rsrc(p.part_ml + static_cast<int64_t>(base) * kRows * 2, extent * kRows * 2 * 4);
        const __amdgpu_buffer_rsrc_t po =
            dev_rsrc(p.part_o + static_cast<int64_t>(base) * kRows * kD, extent * kRows * kD * 4);
        f32x2 ml[8];
        f32x4 ov[8][2];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          ml[j] = f32x2{-INFINITY, 0.f};
          ov[j][0] = ov[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (j < n) {
            const int prow = j * stride * kRows + row;
            ml[j] = ld_dev_b64(pm, prow * 8);
            ov[j][0] = ld_dev_b128(po, (prow * kD + 4 * oc) * 4);
            ov[j][1] = ld_dev_b128(po, (prow * kD + 4 * oc) * 4 + 128);
          }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; ++j) mx = fmaxf(mx, ml[j][0]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float e = (ml[j][0] == -INFINITY) ? 0.f : fast_exp2((ml[j][0] - mx) * p.c);
          den2 = fmaf(ml[j][1], e, den2);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            sum[q] = fmaf(e, ov[j][0][q], sum[q]);
            sum[4 + q] = fmaf(e, ov[j][1][q], sum[4 + q]);
          }
        }
        return mx;
      };
      // level 1: the group's partials, published as the group's partial in its first slot
      const int gbase = slot0 + 8 * grp;
      if (row_thread) {
        const float m_g = merge8(gbase, 1, min(8, s_used - 8 * grp));
        const __amdgpu_buffer_rsrc_t po = dev_rsrc(p.part_o + static_cast<int64_t>(gbase) * kRows * kD, kRows * kD * 4);
        const int off = (row * kD + 4 * oc) * 4;
        st_dev_b128(po, off, f32x4{sum[0], sum[1], sum[2], sum[3]});
        st_dev_b128(po, off + 128, f32x4{sum[4], sum[5], sum[6], sum[7]});
        if (oc == 0) {
          const __amdgpu_buffer_rsrc_t pm = dev_rsrc(p.part_ml + static_cast<int64_t>(gbase) * kRows * 2, kRows * 2 * 4);
          st_dev_b64(pm, row * 8, f32x2{m_g, den2});
        }
      }
      wait_vmcnt<0>();  // the group's partial is complete (visible at device scope)
      __syncthreads();  // every thread has read the group's flag
      if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int is_last = (prev == static_cast<uint32_t>(ngrp - 1));
        if (is_last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag2 = is_last;
      }
      __syncthreads();
      if (!*flag2 || !row_thread) return;
      // level 2: the groups' partials, in group order
      merge8(slot0, 8, ngrp);
      DA_STAMP(45, tid == 0);
      const float inv = den2 > 0.f ? 1.0f / den2 : 0.f;
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = (t_row < b) ? sum[j] * inv : 0.f;
      store_out8(out_row, x);
      DA_STAMP(46, tid == 0);
      return;
    }
  }
  int* last = reinterpret_cast<int*>(smem + kOffFlag);
  if (tid == 0) {
    uint32_t* ctr = p.counters + kCounterStride * rg;
    const uint32_t prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int is_last = (prev == static_cast<uint32_t>(s_used - 1));
    if (is_last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *last = is_last;
  }
  __syncthreads();
  DA_STAMP(44, tid == 0);
  if (!*last || !row_thread) return;

  // Thread (row, oc) merges its row's S partials (the splits this request used) in
  // split order.  Memory round trips dominate here, so every load of a chunk of
  // splits is issued before its first use: one round trip when S <= kChunk.
  const int S = s_used;
  const __amdgpu_buffer_rsrc_t pm = dev_rsrc(p.part_ml + static_cast<int64_t>(slot0) * kRows * 2, S * kRows * 2 * 4);
  const __amdgpu_buffer_rsrc_t po = dev_rsrc(p.part_o + static_cast<int64_t>(slot0) * kRows * kD, S * kRows * kD * 4);
  constexpr int kChunk = 8;
  float den = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  if (S <= kChunk) {
    // one chunk: the maximum over all splits first, then the weighted sums
    f32x2 ml[kChunk];
    f32x4 ov[kChunk][2];
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      ml[j] = f32x2{-INFINITY, 0.f};
      ov[j][0] = ov[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (j < S) {
        const int prow = j * kRows + row;
        ml[j] = ld_dev_b64(pm, prow * 8);
        ov[j][0] = ld_dev_b128(po, (prow * kD + 4 * oc) * 4);
        ov[j][1] = ld_dev_b128(po, (prow * kD + 4 * oc) * 4 + 128);
      }
    }
    float m_all = -INFINITY;
#pragma unroll
    for (int j = 0; j < kChunk; ++j) m_all = fmaxf(m_all, ml[j][0]);
    DA_STAMP(45, tid == 0);
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      // split weight exp2(c (m_s - M)); a split that saw no key (m = -inf) has weight 0
      const float e = (ml[j][0] == -INFINITY) ? 0.f : fast_exp2((ml[j][0] - m_all) * p.c);
      den = fmaf(ml[j][1], e, den);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[q] = fmaf(e, ov[j][0][q], acc[q]);
        acc[4 + q] = fmaf(e, ov[j][1][q], acc[4 + q]);
      }
    }
  } else {
    // More splits (up to 64): chunks of 8 in split order, each loaded whole (one round
    // trip) and merged with a running maximum -- when a chunk raises it, what has been
    // summed so far is rescaled.  The loads are unconditional: past the last split the
    // buffer's range check returns zeros, which the mask gives weight 0.
    f32x2 ml[kChunk];
    f32x4 ov[kChunk][2];
    float m_run_all = -INFINITY;
    for (int s0 = 0; s0 < S; s0 += kChunk) {
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        const int prow = (s0 + j) * kRows + row;
        ml[j] = ld_dev_b64(pm, prow * 8);
        ov[j][0] = ld_dev_b128(po, (prow * kD + 4 * oc) * 4);
        ov[j][1] = ld_dev_b128(po, (prow * kD + 4 * oc) * 4 + 128);
      }
      float mj[kChunk];
      float mc = -INFINITY;
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        mj[j] = s0 + j < S ? ml[j][0] : -INFINITY;
        mc = fmaxf(mc, mj[j]);
      }
      const float mn = fmaxf(m_run_all, mc);
      // nothing summed yet (running maximum -inf): the sums are zero, scale 0
      const float sc = (m_run_all == -INFINITY) ? 0.f : fast_exp2((m_run_all - mn) * p.c);
      den *= sc;
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] *= sc;
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        const float e = (mj[j] == -INFINITY) ? 0.f : fast_exp2((mj[j] - mn) * p.c);
        den = fmaf(ml[j][1], e, den);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[q] = fmaf(e, ov[j][0][q], acc[q]);
          acc[4 + q] = fmaf(e, ov[j][1][q], acc[4 + q]);
        }
      }
      m_run_all = mn;
    }
    DA_STAMP(45, tid == 0);
  }
  // den > 0 whenever there is a key (always with the block's own keys, in split 0)
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (t_row < b) ? acc[j] * inv : 0.f;
  store_out8(out_row, x);
  DA_STAMP(46, tid == 0);
}

// ---------------------------------------------------------------------------------
// standalone q/k RMSNorm + NeoX RoPE, in place on the packed rows
// ---------------------------------------------------------------------------------
// Workgroup (x, y): tokens 8x .. 8x+7, and rows 32y .. 32y+31 of their list of
// (token, q-or-k head) rows; 8 threads per row, 16 bytes each.  The row values,
// norm weights and positions are loaded first; the rotation table of the 8 tokens
// goes through LDS.  The arithmetic is the attention kernel's prologue
// (rope_cos_sin, norm_rope_row), so these rows are bit-identical to the q/k rows
// that kernel builds from the same inputs.
constexpr int kNrTokens = 8;
constexpr int kNrThreads = 256;
constexpr int kNrRows = kNrThreads / 8;

struct NrParams {
  uint16_t* qkv;
  int64_t qkv_stride;
  const void* positions;
  const uint16_t* wq;
  const uint16_t* wk;
  int32_t N, Hq, Hkv;
  float eps;
  Rope rope;
};

template <bool POS64>
__global__ __launch_bounds__(kNrThreads) void qk_norm_rope_kernel(const NrParams p) {
  __shared__ float2 cs[kNrTokens * 32];
  const int tid = threadIdx.x, u = tid & 7;
  const int t0 = blockIdx.x * kNrTokens;
  const int nt = min(kNrTokens, p.N - t0);
  const int heads = p.Hq + p.Hkv;
  const int rr = blockIdx.y * kNrRows + (tid >> 3);  // row of this workgroup's (token, head) list
  const int t = rr / heads, h = rr - t * heads;
  const bool live = t < nt;
  uint16_t* row = p.qkv + static_cast<int64_t>(t0 + t) * p.qkv_stride + h * kD + 8 * u;
  u32x4 raw = {0u, 0u, 0u, 0u}, wraw = {0u, 0u, 0u, 0u};
  if (live) {
    raw = ld16(row);
    wraw = ld16((h < p.Hq ? p.wq : p.wk) + 8 * u);
  }
  int64_t pos = 0;
  if (tid < nt * 32)
    pos = POS64 ? static_cast<const int64_t*>(p.positions)[t0 + (tid >> 5)]
                : static_cast<int64_t>(static_cast<const int32_t*>(p.positions)[t0 + (tid >> 5)]);
  if (tid < nt * 32) cs[tid] = rope_cos_sin(pos, tid & 31, p.rope);
  __syncthreads();
  if (live) {
    float x[8];
    unpack8(raw, x);
    norm_rope_row(x, wraw, p.eps, cs + t * 32, u);
    *reinterpret_cast<u32x4*>(row) = pack8(x);
  }
}

// ---------------------------------------------------------------------------------
// append the block's K/V to the pool (the path the fused op replaces)
// ---------------------------------------------------------------------------------
// Workgroup (r, g): 8 tokens x (K, V) x 8 lanes of 16 bytes.  Token t < b of
// request r goes to logical slot L + t of its paged row.  A request whose L + b
// does not fit its row, and a token whose page id is out of range, is skipped and
// flagged (writing elsewhere would corrupt the pool).
constexpr int kApThreads = kMaxT * 2 * 8;

__global__ __launch_bounds__(kApThreads) void kv_append_kernel(const Params p) {
  const int r = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, t = tid >> 4, is_v = (tid >> 3) & 1, u = tid & 7;
  const int T = p.T;
  const int L = p.ctx_lens[r];
  int b = p.blk_lens ? p.blk_lens[r] : T;
  if (b < 1 || b > T) {
    if (tid == 0 && g == 0) flag(p.status, DA_FLAG_BLOCK_LEN);
    b = b < 1 ? 1 : T;
  }
  // L + b could overflow for a length near INT_MAX: compare against the room left instead
  if (L < 0 || L > p.pt_stride * kPage - b) {
    if (tid == 0 && g == 0) flag(p.status, DA_FLAG_CONTEXT_LEN);
    return;
  }
  if (t >= b) return;
  const int logical = L + t;
  const int id = p.page_table[static_cast<int64_t>(r) * p.pt_stride + logical / kPage];
  if (id < 0 || id >= p.num_pages) {
    flag(p.status, DA_FLAG_PAGE_ID);
    return;
  }
  const int col = (is_v ? p.Hq + p.Hkv + g : p.Hq + g) * kD + 8 * u;
  const u32x4 val = ld16(p.qkv + static_cast<int64_t>(r * T + t) * p.qkv_stride + col);
  uint16_t* pool = const_cast<uint16_t*>(is_v ? p.vpool : p.kpool);
  *reinterpret_cast<u32x4*>(pool + static_cast<int64_t>(id) * p.page_stride +
                            (static_cast<int64_t>(g) * kPage + logical % kPage) * kD + 8 * u) = val;
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
// per split that is a multiple of the 8 waves; at most kMaxSplits splits.  A
// problem so small that a split would hold at most 4 pages' worth gets splits of
// 4 pages (half the waves idle): a compute unit takes only a few of a workgroup's
// page loads at a time, so twice the workgroups fetch the pages sooner, and the
// combine then has no more than twice the partials to read.
Plan make_plan(int R, int Hkv, int stride) {
  constexpr int kTargetWorkgroups = 256;
  if (stride <= 0) return {1, 1};
  const int64_t units = static_cast<int64_t>(R) * Hkv * stride;
  int ps = static_cast<int>((units + kTargetWorkgroups - 1) / kTargetWorkgroups);
  ps = ps <= 4 ? 4 : (ps + kWaves - 1) / kWaves * kWaves;
  if (ps > kMaxPagesPerSplit) ps = kMaxPagesPerSplit;
  int S = (stride + ps - 1) / ps;
  if (S > kMaxSplits) {
    ps = (stride + kMaxSplits - 1) / kMaxSplits;
    ps = (ps + kWaves - 1) / kWaves * kWaves;
    S = (stride + ps - 1) / ps;
  }
  return {S, ps};  // S <= 64, ps <= 512 (kMaxStride <= 64 * 256)
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct WsLayout {
  size_t counters, part_o, part_ml, total;
};

// Counters first (counter_bytes, at least R * Hkv lines of 256 bytes), then the fp32
// partial outputs and the (max, sum) pairs, each region 256-byte aligned.
WsLayout ws_layout_after(size_t counter_bytes, int R, int Hkv, int S) {
  WsLayout l;
  l.counters = 0;
  l.part_o = align256(counter_bytes);
  l.part_ml = l.part_o + align256(static_cast<size_t>(R) * Hkv * S * kRows * kD * 4);
  l.total = l.part_ml + align256(static_cast<size_t>(R) * Hkv * S * kRows * 2 * 4);
  return l;
}

WsLayout ws_layout(int R, int Hkv, int S) {
  return ws_layout_after(static_cast<size_t>(R) * Hkv * kCounterStride * 4, R, Hkv, S);
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned_to(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

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

// Byte extents of the arrays an attention call reads (ins) and of the rows it writes.
struct Extent {
  const void* p;
  size_t n;
  const char* name;
};
struct Extents {
  size_t out_n;
  Extent ins[6];
};

Extents extents(const Common& a) {
  const int64_t rows = static_cast<int64_t>(a.R) * a.T;
  const int64_t width = static_cast<int64_t>(a.Hq + 2 * a.Hkv) * kD;
  const size_t qkv_n = static_cast<size_t>(((rows - 1) * a.qkv_row_stride + width) * 2);
  const size_t pool_n = a.page_table_stride > 0
      ? static_cast<size_t>(((static_cast<int64_t>(a.num_pages) - 1) * a.pool_page_stride + static_cast<int64_t>(a.Hkv) * kPage * kD) * 2)
      : 0;
  const size_t pt_n = static_cast<size_t>(a.R) * a.page_table_stride * 4;
  const size_t r_n = static_cast<size_t>(a.R) * 4;
  return Extents{static_cast<size_t>(((rows - 1) * a.out_row_stride + a.Hq * kD) * 2),
                 {{a.qkv, qkv_n, "qkv"}, {a.k_pool, pool_n, "k_pool"}, {a.v_pool, pool_n, "v_pool"},
                  {a.page_table, pt_n, "page_table"}, {a.context_lens, r_n, "context_lens"},
                  {a.block_lens, r_n, "block_lens"}}};
}

int check_sizes(int R, int T, int Hq, int Hkv, int head_dim, int page_size, int stride) {
  if (head_dim != kD) return fail(DA_EUNSUPPORTED, "head_dim must be 64");
  if (page_size != kPage) return fail(DA_EUNSUPPORTED, "page_size must be 64");
  if (R < 1 || R > DA_MAX_REQUESTS) return fail(DA_EINVAL, "num_requests must be in [1, 8]");
  if (T < 1 || T > DA_MAX_TOKENS) return fail(DA_EINVAL, "tokens_per_block must be in [1, 8]");
  if (Hkv < 1 || Hkv > DA_MAX_KV_HEADS) return fail(DA_EINVAL, "num_kv_heads must be in [1, 16]");
  if (Hq != kG * Hkv) return fail(DA_EUNSUPPORTED, "num_q_heads must be 6 * num_kv_heads");
  if (stride < 0) return fail(DA_EINVAL, "page_table_stride must be >= 0");
  if (stride > kMaxStride) return fail(DA_EINVAL, "page_table_stride above 16384 pages (1M tokens) is not supported");
  return DA_OK;
}

// Every check of the attention arguments except those of the workspace.
int validate_args(const Common& a) {
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
  if (!aligned_to(a.page_table, 4) || !aligned_to(a.context_lens, 4) || !aligned_to(a.block_lens, 4) ||
      !aligned_to(a.status_word, 4))
    return fail(DA_EINVAL, "page_table, context_lens, block_lens and status_word must be 4-byte aligned");
  if (!(std::isfinite(a.scale) && a.scale > 0.f)) return fail(DA_EINVAL, "scale must be finite and > 0");
  const Extents x = extents(a);
  for (const Extent& in : x.ins)
    if (overlaps(a.out, x.out_n, in.p, in.n)) return fail(DA_EINVAL, std::string("out overlaps ") + in.name);
  if (a.status_word && overlaps(a.status_word, 4, a.out, x.out_n)) return fail(DA_EINVAL, "status_word overlaps out");
  return DA_OK;
}

// validate_args, then the caller's workspace: present, large enough, 256-byte aligned,
// overlapping no input, out or the status word.
int validate(const Common& a, size_t need_ws) {
  int rc = validate_args(a);
  if (rc != DA_OK) return rc;
  if (!a.workspace || a.workspace_bytes < need_ws)
    return fail(DA_EWORKSPACE, "workspace missing or smaller than drafter_attn_workspace_bytes()");
  if (reinterpret_cast<uintptr_t>(a.workspace) & 255u) return fail(DA_EWORKSPACE, "workspace must be 256-byte aligned");
  const Extents x = extents(a);
  for (const Extent& in : x.ins)
    if (overlaps(a.workspace, need_ws, in.p, in.n)) return fail(DA_EINVAL, std::string("workspace overlaps ") + in.name);
  if (overlaps(a.out, x.out_n, a.workspace, need_ws)) return fail(DA_EINVAL, "out overlaps workspace");
  if (a.status_word && overlaps(a.status_word, 4, a.workspace, need_ws))
    return fail(DA_EINVAL, "status_word overlaps workspace");
  return DA_OK;
}

Params make_params(const Common& a, const Plan& plan, const WsLayout& l) {
  Params p;
  std::memset(&p, 0, sizeof(p));
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
  // the balanced plan is taken when Ps >= 32 (4 pages per wave) and its splits of Pb
  // pages (a multiple of 8) hold at most M = 3 Ps / 4 (rounded down to a multiple of
  // 8), i.e. ceil(N / (R (S-1))) and ceil(max npg / 32) are both at most M: a smaller
  // saving does not pay for the extra round trip.  (A build with DA_STATIC_PLAN_ONLY
  // defined keeps the static plan everywhere: the reference the scheduling is measured
  // against.)
#ifndef DA_STATIC_PLAN_ONLY
  if (plan.S > 1 && plan.Ps >= 4 * kWaves) {
#else
  if (false) {
#endif
    const int M = 3 * plan.Ps / 4 / kWaves * kWaves;
    p.bal_n = a.R * (plan.S - 1) * M;
    p.bal_npg = kMaxReqSplits * M;
  }
  p.c = static_cast<float>(static_cast<double>(a.scale) * 1.4426950408889634);  // log2(e)
  return p;
}

template <int NT, bool QK, bool P64, bool OWN>
int launch_t(const Params& p, const Plan& plan, hipStream_t stream) {
  dim3 grid(plan.S, p.Hkv, p.R);
  // The length-aware schedule is compiled in only where the plan leaves it room (its
  // code costs the static path 0.1-0.8 us on the 32k workload even where it is never
  // taken), and the two-level combine only into the kernel of plans with more than
  // kTwoLevel splits (its code moves the page loop's scheduling: +0.1-0.25 us elsewhere).
  const bool many = plan.S > kTwoLevel;
  if (p.bal_n > 0) {
    if (many)
      hipLaunchKernelGGL((drafter_attn_kernel<NT, QK, P64, OWN, true, true>), grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((drafter_attn_kernel<NT, QK, P64, OWN, true, false>), grid, dim3(kThreads), 0, stream, p);
  } else {
    if (many)
      hipLaunchKernelGGL((drafter_attn_kernel<NT, QK, P64, OWN, false, true>), grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((drafter_attn_kernel<NT, QK, P64, OWN, false, false>), grid, dim3(kThreads), 0, stream, p);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DA_ELAUNCH, std::string("launch failed: ") + hipGetErrorString(e));
  return DA_OK;
}

template <bool QK, bool P64, bool OWN = true>
int launch_nt(const Params& p, const Plan& plan, hipStream_t stream) {
  const int nt = (kG * p.T + 15) / 16;
  if (nt == 1) return launch_t<1, QK, P64, OWN>(p, plan, stream);
  if (nt == 2) return launch_t<2, QK, P64, OWN>(p, plan, stream);
  return launch_t<3, QK, P64, OWN>(p, plan, stream);
}

template <bool P64>
int launch_norm_rope(const NrParams& p, hipStream_t stream) {
  dim3 grid((p.N + kNrTokens - 1) / kNrTokens, (kNrTokens * (p.Hq + p.Hkv) + kNrRows - 1) / kNrRows);
  hipLaunchKernelGGL((qk_norm_rope_kernel<P64>), grid, dim3(kNrThreads), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DA_ELAUNCH, std::string("launch failed: ") + hipGetErrorString(e));
  return DA_OK;
}

int check_yarn(const da_yarn* y, float rope_base) {
  if (!y) return DA_OK;
  if (!(std::isfinite(y->factor) && y->factor >= 1.f)) return fail(DA_EINVAL, "yarn factor must be finite and >= 1");
  if (y->original_max_position < 1) return fail(DA_EINVAL, "yarn original_max_position must be >= 1");
  if (!(std::isfinite(y->alpha) && std::isfinite(y->beta) && y->alpha >= 0.f && y->beta > y->alpha))
    return fail(DA_EINVAL, "yarn alpha and beta must be finite with 0 <= alpha < beta");
  if (y->ramp != DA_YARN_RAMP_TURNS && y->ramp != DA_YARN_RAMP_INDEX && y->ramp != DA_YARN_RAMP_INDEX_UNROUNDED)
    return fail(DA_EINVAL, "yarn ramp must be DA_YARN_RAMP_TURNS, DA_YARN_RAMP_INDEX or DA_YARN_RAMP_INDEX_UNROUNDED");
  if (!(std::isfinite(y->mscale) && y->mscale >= 0.f))
    return fail(DA_EINVAL, "yarn mscale must be finite and >= 0 (0: the default temperature)");
  if (y->ramp != DA_YARN_RAMP_TURNS && !(rope_base > 1.f))
    return fail(DA_EINVAL, "yarn ramps in the pair index need rope_base > 1 (frequencies falling with the pair)");
  return DA_OK;
}

// The rotation's parameters from the host arguments.  A YaRN factor of 1 with the
// default factor on q and k is the plain rotation (taken as such, so it gives the
// same bits).  For the ramps in the pair index, the pair that turns rho times over
// the original context L is i(rho) = 32 ln(L / (2 pi rho)) / ln(base) (f_i =
// base^(-2i/64) solved for L f_i / (2 pi) = rho); the ramp runs from lo = i(beta)
// down-rounded to hi = i(alpha) up-rounded (or unrounded), both clamped to the
// pairs 0..31, and is a step after lo where they meet.
Rope make_rope(float rope_base, const da_yarn* y) {
  Rope r;
  std::memset(&r, 0, sizeof(r));
  r.log2_base = std::log2(static_cast<double>(rope_base));
  r.inv_s = 1.0;
  r.mscale = 1.f;
  if (!y) return r;
  const double s = y->factor;
  const float m = y->mscale > 0.f ? y->mscale : static_cast<float>(0.1 * std::log(s) + 1.0);
  if (y->factor == 1.f && m == 1.f) return r;
  r.yarn = 1;
  r.inv_s = 1.0 / s;
  r.mscale = m;
  const double L = y->original_max_position, alpha = y->alpha, beta = y->beta;
  constexpr double kTwoPi = 6.283185307179586;
  if (y->ramp == DA_YARN_RAMP_TURNS) {
    r.turn_scale = L / kTwoPi;
    r.start = alpha;
    r.inv_ramp = 1.0 / (beta - alpha);
    return r;
  }
  const double ln_base = std::log(static_cast<double>(rope_base));
  auto pair_at = [&](double rho) {
    const double i = rho > 0.0 ? 32.0 * std::log(L / (kTwoPi * rho)) / ln_base : INFINITY;
    return std::fmin(std::fmax(i, 0.0), 31.0);
  };
  double lo = pair_at(beta), hi = pair_at(alpha);
  if (y->ramp == DA_YARN_RAMP_INDEX) {
    lo = std::floor(lo);
    hi = std::ceil(hi);
  }
  r.yarn = 2;
  if (hi > lo) {  // gamma = clamp((hi - i) / (hi - lo))
    r.start = -hi;
    r.inv_ramp = 1.0 / (hi - lo);
  } else {  // gamma = 1 for pairs i <= lo, else 0
    r.start = -(std::floor(lo) + 0.5);
    r.inv_ramp = 0x1p900;
  }
  return r;
}

// The qknorm arguments (positions, norm weights, eps, base, YaRN parameters), and that
// neither out nor the workspace (ws_n bytes at ws; none when ws is NULL) overlaps them.
struct QkArgs {
  const void* positions;
  int32_t positions_dtype;
  const void* wq;
  const void* wk;
  float eps, rope_base;
  const da_yarn* yarn;
};

int validate_qk(const Common& a, const QkArgs& q, const void* ws, size_t ws_n) {
  if (!q.positions || !q.wq || !q.wk) return fail(DA_EINVAL, "positions, q_norm_weight and k_norm_weight must be non-NULL");
  if (q.positions_dtype != DA_POS_INT32 && q.positions_dtype != DA_POS_INT64)
    return fail(DA_EINVAL, "positions_dtype must be DA_POS_INT32 or DA_POS_INT64");
  if (!aligned_to(q.positions, q.positions_dtype == DA_POS_INT64 ? 8 : 4))
    return fail(DA_EINVAL, "positions must be aligned to its element size");
  if (!(std::isfinite(q.eps) && q.eps >= 0.f)) return fail(DA_EINVAL, "eps must be finite and >= 0");
  if (!(std::isfinite(q.rope_base) && q.rope_base > 0.f)) return fail(DA_EINVAL, "rope_base must be finite and > 0");
  const int rc = check_yarn(q.yarn, q.rope_base);
  if (rc != DA_OK) return rc;
  if (!aligned16(q.wq) || !aligned16(q.wk)) return fail(DA_EINVAL, "q_norm_weight and k_norm_weight must be 16-byte aligned");
  const size_t out_n = extents(a).out_n;
  const size_t pos_n = static_cast<size_t>(a.R) * a.T * (q.positions_dtype == DA_POS_INT64 ? 8 : 4);
  if (overlaps(a.out, out_n, q.positions, pos_n) || overlaps(a.out, out_n, q.wq, kD * 2) ||
      overlaps(a.out, out_n, q.wk, kD * 2))
    return fail(DA_EINVAL, "out overlaps positions or a norm weight");
  if (overlaps(ws, ws_n, q.positions, pos_n) || overlaps(ws, ws_n, q.wq, kD * 2) || overlaps(ws, ws_n, q.wk, kD * 2))
    return fail(DA_EINVAL, "workspace overlaps positions or a norm weight");
  return DA_OK;
}

int launch_qk(Params p, const Plan& plan, const QkArgs& q, void* stream) {
  p.positions = q.positions;
  p.wq = static_cast<const uint16_t*>(q.wq);
  p.wk = static_cast<const uint16_t*>(q.wk);
  p.eps = q.eps;
  p.rope = make_rope(q.rope_base, q.yarn);
  g_last_error.clear();
  hipStream_t st = static_cast<hipStream_t>(stream);
  return q.positions_dtype == DA_POS_INT64 ? launch_nt<true, true>(p, plan, st) : launch_nt<true, false>(p, plan, st);
}

}  // namespace

// ---------------------------------------------------------------------------------
// scratch of the no-allocation entry point
// ---------------------------------------------------------------------------------
// Device memory that the library holds for callers that cannot allocate: the
// arrival counters (a fixed region for the largest R * Hkv, so that calls of any
// size find theirs at zero) and the split partials.  Every GPU the library runs on
// holds its own copy until the process ends.  In host code `scratch` names a
// host-side stand-in: its device address comes from hipGetSymbolAddress, once per
// device, and only that address is handed to kernels.
constexpr size_t kScratchBytes = DA_NOALLOC_SCRATCH_BYTES;
constexpr size_t kScratchCounterBytes = static_cast<size_t>(DA_MAX_REQUESTS) * DA_MAX_KV_HEADS * kCounterStride * 4;
static_assert(kScratchCounterBytes % 256 == 0, "scratch counters region");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];  // device address of `scratch` on each device, once set up

// The current device's scratch.  The first call on a device looks up its address and
// clears its counters on `stream` (ordered before the kernels that follow); that call
// must not be under stream capture.  Afterwards every call leaves the counters zero.
int scratch_of_current_device(void* stream, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DA_ELAUNCH, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(DA_ELAUNCH, "device ordinal above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cap);
    if (e != hipSuccess) return fail(DA_ELAUNCH, std::string("hipStreamIsCapturing: ") + hipGetErrorString(e));
    if (cap != hipStreamCaptureStatusNone)
      return fail(DA_EINVAL, "the first drafter_attn_qknorm_noalloc call on a device sets up its scratch and must "
                             "not be captured");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(DA_ELAUNCH, std::string("hipGetSymbolAddress: ") + hipGetErrorString(e));
    e = hipMemsetAsync(p, 0, kScratchCounterBytes, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(DA_ELAUNCH, std::string("clearing the scratch counters: ") + hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *ptr = g_scratch_dev[dev];
  return DA_OK;
}

}  // namespace

extern "C" {

size_t drafter_attn_workspace_bytes(int32_t num_requests, int32_t tokens_per_block, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t page_table_stride) {
  if (check_sizes(num_requests, tokens_per_block, num_q_heads, num_kv_heads, head_dim, kPage, page_table_stride) !=
      DA_OK)
    return 0;
  const Plan plan = make_plan(num_requests, num_kv_heads, page_table_stride);
  return ws_layout(num_requests, num_kv_heads, plan.S).total;
}

int drafter_attn_plan(int32_t num_requests, int32_t num_kv_heads, int32_t page_table_stride,
                      int32_t* num_splits, int32_t* pages_per_split) {
  if (num_requests < 1 || num_requests > DA_MAX_REQUESTS || num_kv_heads < 1 ||
      num_kv_heads > DA_MAX_KV_HEADS || page_table_stride < 0 || page_table_stride > kMaxStride)
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
                                                   head_dim, page_table_stride);
  int rc = validate(a, need);
  if (rc != DA_OK) return rc;
  const Plan plan = make_plan(num_requests, num_kv_heads, page_table_stride);
  Params p = make_params(a, plan, ws_layout(a.R, a.Hkv, plan.S));
  g_last_error.clear();
  return launch_nt<false, false>(p, plan, static_cast<hipStream_t>(stream));
}

int drafter_attn_qknorm_yarn(const void* qkv, int64_t qkv_row_stride, const void* k_pool, const void* v_pool,
                             int64_t pool_page_stride, int32_t num_pages, const int32_t* page_table,
                             int32_t page_table_stride, const int32_t* context_lens, const int32_t* block_lens,
                             int32_t num_requests, int32_t tokens_per_block, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t page_size, float scale,
                             const void* positions, int32_t positions_dtype, const void* q_norm_weight,
                             const void* k_norm_weight, float eps, float rope_base, const da_yarn* yarn,
                             void* workspace, size_t workspace_bytes, void* out, int64_t out_row_stride,
                             int32_t* status_word, void* stream) {
  const Common a{qkv, qkv_row_stride, k_pool, v_pool, pool_page_stride, num_pages, page_table, page_table_stride,
                 context_lens, block_lens, num_requests, tokens_per_block, num_q_heads, num_kv_heads, head_dim,
                 page_size, scale, workspace, workspace_bytes, out, out_row_stride, status_word, stream};
  const QkArgs q{positions, positions_dtype, q_norm_weight, k_norm_weight, eps, rope_base, yarn};
  const size_t need = drafter_attn_workspace_bytes(num_requests, tokens_per_block, num_q_heads, num_kv_heads,
                                                   head_dim, page_table_stride);
  int rc = validate(a, need);
  if (rc != DA_OK) return rc;
  rc = validate_qk(a, q, workspace, need);
  if (rc != DA_OK) return rc;
  const Plan plan = make_plan(num_requests, num_kv_heads, page_table_stride);
  return launch_qk(make_params(a, plan, ws_layout(num_requests, num_kv_heads, plan.S)), plan, q, stream);
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
  return drafter_attn_qknorm_yarn(qkv, qkv_row_stride, k_pool, v_pool, pool_page_stride, num_pages, page_table,
                                  page_table_stride, context_lens, block_lens, num_requests, tokens_per_block,
                                  num_q_heads, num_kv_heads, head_dim, page_size, scale, positions,
                                  positions_dtype, q_norm_weight, k_norm_weight, eps, rope_base, nullptr,
                                  workspace, workspace_bytes, out, out_row_stride, status_word, stream);
}

int drafter_attn_qknorm_noalloc(const void* qkv, int64_t qkv_row_stride, const void* k_pool, const void* v_pool,
                                int64_t pool_page_stride, int32_t num_pages, const int32_t* page_table,
                                int32_t page_table_stride, const int32_t* context_lens, const int32_t* block_lens,
                                int32_t num_requests, int32_t tokens_per_block, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t page_size, float scale,
                                const void* positions, int32_t positions_dtype, const void* q_norm_weight,
                                const void* k_norm_weight, float eps, float rope_base, void* out,
                                int64_t out_row_stride, int32_t* status_word, void* stream) {
  Common a{qkv, qkv_row_stride, k_pool, v_pool, pool_page_stride, num_pages, page_table, page_table_stride,
           context_lens, block_lens, num_requests, tokens_per_block, num_q_heads, num_kv_heads, head_dim,
           page_size, scale, nullptr, 0, out, out_row_stride, status_word, stream};
  const QkArgs q{positions, positions_dtype, q_norm_weight, k_norm_weight, eps, rope_base, nullptr};
  // every host check first: a refused call touches no device
  int rc = validate_args(a);
  if (rc != DA_OK) return rc;
  rc = validate_qk(a, q, nullptr, 0);
  if (rc != DA_OK) return rc;
  const Plan plan = make_plan(num_requests, num_kv_heads, page_table_stride);
  const WsLayout l = ws_layout_after(kScratchCounterBytes, num_requests, num_kv_heads, plan.S);
  if (l.total > kScratchBytes)
    return fail(DA_EWORKSPACE, "these sizes need " + std::to_string(l.total) + " bytes of scratch, above the " +
                                   std::to_string(kScratchBytes) + " the no-allocation entry point holds");
  rc = scratch_of_current_device(stream, &a.workspace);
  if (rc != DA_OK) return rc;
  a.workspace_bytes = kScratchBytes;
  return launch_qk(make_params(a, plan, l), plan, q, stream);
}

int drafter_qk_norm_rope_yarn(void* qkv, int64_t qkv_row_stride, int32_t num_tokens, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, const void* positions,
                              int32_t positions_dtype, const void* q_norm_weight, const void* k_norm_weight,
                              float eps, float rope_base, const da_yarn* yarn, void* stream) {
  if (head_dim != kD) return fail(DA_EUNSUPPORTED, "head_dim must be 64");
  if (num_kv_heads < 1 || num_kv_heads > DA_MAX_KV_HEADS) return fail(DA_EINVAL, "num_kv_heads must be in [1, 16]");
  if (num_q_heads != kG * num_kv_heads) return fail(DA_EUNSUPPORTED, "num_q_heads must be 6 * num_kv_heads");
  if (num_tokens < 1 || num_tokens > DA_MAX_NORM_TOKENS) return fail(DA_EINVAL, "num_tokens must be in [1, 65536]");
  if (!qkv || !positions || !q_norm_weight || !k_norm_weight)
    return fail(DA_EINVAL, "qkv, positions, q_norm_weight and k_norm_weight must be non-NULL");
  const int64_t width = static_cast<int64_t>(num_q_heads + 2 * num_kv_heads) * kD;
  if (qkv_row_stride < width) return fail(DA_EINVAL, "qkv_row_stride must be >= (Hq + 2*Hkv) * 64");
  if (qkv_row_stride % 8) return fail(DA_EINVAL, "qkv_row_stride must be a multiple of 8 elements");
  if (!aligned16(qkv) || !aligned16(q_norm_weight) || !aligned16(k_norm_weight))
    return fail(DA_EINVAL, "qkv, q_norm_weight and k_norm_weight must be 16-byte aligned");
  if (positions_dtype != DA_POS_INT32 && positions_dtype != DA_POS_INT64)
    return fail(DA_EINVAL, "positions_dtype must be DA_POS_INT32 or DA_POS_INT64");
  if (!aligned_to(positions, positions_dtype == DA_POS_INT64 ? 8 : 4))
    return fail(DA_EINVAL, "positions must be aligned to its element size");
  if (!(std::isfinite(eps) && eps >= 0.f)) return fail(DA_EINVAL, "eps must be finite and >= 0");
  if (!(std::isfinite(rope_base) && rope_base > 0.f)) return fail(DA_EINVAL, "rope_base must be finite and > 0");
  const int rc = check_yarn(yarn, rope_base);
  if (rc != DA_OK) return rc;
  const size_t qkv_n = static_cast<size_t>(((num_tokens - 1) * qkv_row_stride + width) * 2);
  const size_t pos_n = static_cast<size_t>(num_tokens) * (positions_dtype == DA_POS_INT64 ? 8 : 4);
  if (overlaps(qkv, qkv_n, positions, pos_n) || overlaps(qkv, qkv_n, q_norm_weight, kD * 2) ||
      overlaps(qkv, qkv_n, k_norm_weight, kD * 2))
    return fail(DA_EINVAL, "qkv (written in place) overlaps positions or a norm weight");
  NrParams p;
  std::memset(&p, 0, sizeof(p));
  p.qkv = static_cast<uint16_t*>(qkv);
  p.qkv_stride = qkv_row_stride;
  p.positions = positions;
  p.wq = static_cast<const uint16_t*>(q_norm_weight);
  p.wk = static_cast<const uint16_t*>(k_norm_weight);
  p.N = num_tokens;
  p.Hq = num_q_heads;
  p.Hkv = num_kv_heads;
  p.eps = eps;
  p.rope = make_rope(rope_base, yarn);
  g_last_error.clear();
  hipStream_t st = static_cast<hipStream_t>(stream);
  return positions_dtype == DA_POS_INT64 ? launch_norm_rope<true>(p, st) : launch_norm_rope<false>(p, st);
}

int drafter_qk_norm_rope(void* qkv, int64_t qkv_row_stride, int32_t num_tokens, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, const void* positions, int32_t positions_dtype,
                         const void* q_norm_weight, const void* k_norm_weight, float eps, float rope_base,
                         void* stream) {
  return drafter_qk_norm_rope_yarn(qkv, qkv_row_stride, num_tokens, num_q_heads, num_kv_heads, head_dim, positions,
                                   positions_dtype, q_norm_weight, k_norm_weight, eps, rope_base, nullptr, stream);
}

int drafter_paged_attn(const void* qkv, int64_t qkv_row_stride, const void* k_pool, const void* v_pool,
                       int64_t pool_page_stride, int32_t num_pages, const int32_t* page_table,
                       int32_t page_table_stride, const int32_t* kv_lens, const int32_t* block_lens,
                       int32_t num_requests, int32_t tokens_per_block, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t page_size, float scale, void* workspace, size_t workspace_bytes,
                       void* out, int64_t out_row_stride, int32_t* status_word, void* stream) {
  const Common a{qkv, qkv_row_stride, k_pool, v_pool, pool_page_stride, num_pages, page_table, page_table_stride,
                 kv_lens, block_lens, num_requests, tokens_per_block, num_q_heads, num_kv_heads, head_dim,
                 page_size, scale, workspace, workspace_bytes, out, out_row_stride, status_word, stream};
  const size_t need = drafter_attn_workspace_bytes(num_requests, tokens_per_block, num_q_heads, num_kv_heads,
                                                   head_dim, page_table_stride);
  int rc = validate(a, need);
  if (rc != DA_OK) return rc;
  const Plan plan = make_plan(num_requests, num_kv_heads, page_table_stride);
  Params p = make_params(a, plan, ws_layout(a.R, a.Hkv, plan.S));
  g_last_error.clear();
  return launch_nt<false, false, false>(p, plan, static_cast<hipStream_t>(stream));
}

int drafter_kv_append(const void* qkv, int64_t qkv_row_stride, void* k_pool, void* v_pool, int64_t pool_page_stride,
                      int32_t num_pages, const int32_t* page_table, int32_t page_table_stride,
                      const int32_t* context_lens, const int32_t* block_lens, int32_t num_requests,
                      int32_t tokens_per_block, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t page_size, int32_t* status_word, void* stream) {
  int rc = check_sizes(num_requests, tokens_per_block, num_q_heads, num_kv_heads, head_dim, page_size,
                       page_table_stride);
  if (rc != DA_OK) return rc;
  if (!qkv || !k_pool || !v_pool || !page_table || !context_lens)
    return fail(DA_EINVAL, "qkv, k_pool, v_pool, page_table and context_lens must be non-NULL");
  if (page_table_stride < 1) return fail(DA_EINVAL, "page_table_stride must be >= 1 (the block needs a page)");
  if (num_pages < 1) return fail(DA_EINVAL, "num_pages must be >= 1");
  if (pool_page_stride < static_cast<int64_t>(num_kv_heads) * kPage * kD)
    return fail(DA_EINVAL, "pool_page_stride must be >= num_kv_heads * 64 * 64");
  if (pool_page_stride % 8) return fail(DA_EINVAL, "pool_page_stride must be a multiple of 8 elements");
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(qkv))
    return fail(DA_EINVAL, "qkv, k_pool and v_pool must be 16-byte aligned");
  if (!aligned_to(page_table, 4) || !aligned_to(context_lens, 4) || !aligned_to(block_lens, 4) ||
      !aligned_to(status_word, 4))
    return fail(DA_EINVAL, "page_table, context_lens, block_lens and status_word must be 4-byte aligned");
  const int64_t width = static_cast<int64_t>(num_q_heads + 2 * num_kv_heads) * kD;
  if (qkv_row_stride < width) return fail(DA_EINVAL, "qkv_row_stride must be >= (Hq + 2*Hkv) * 64");
  if (qkv_row_stride % 8) return fail(DA_EINVAL, "qkv_row_stride must be a multiple of 8 elements");
  // the pools are written: they must not overlap anything the kernel reads or writes besides themselves
  const int64_t rows = static_cast<int64_t>(num_requests) * tokens_per_block;
  const size_t pool_n = static_cast<size_t>(((static_cast<int64_t>(num_pages) - 1) * pool_page_stride +
                                             static_cast<int64_t>(num_kv_heads) * kPage * kD) * 2);
  const size_t qkv_n = static_cast<size_t>(((rows - 1) * qkv_row_stride + width) * 2);
  const size_t pt_n = static_cast<size_t>(num_requests) * page_table_stride * 4;
  const size_t r_n = static_cast<size_t>(num_requests) * 4;
  const struct { const void* p; size_t n; const char* name; } ins[] = {
      {qkv, qkv_n, "qkv"}, {page_table, pt_n, "page_table"}, {context_lens, r_n, "context_lens"},
      {block_lens, r_n, "block_lens"}, {status_word, 4, "status_word"}};
  for (const auto& in : ins) {
    if (overlaps(k_pool, pool_n, in.p, in.n) || overlaps(v_pool, pool_n, in.p, in.n))
      return fail(DA_EINVAL, std::string("the pool overlaps ") + in.name);
  }
  Params p;
  std::memset(&p, 0, sizeof(p));
  p.qkv = static_cast<const uint16_t*>(qkv);
  p.qkv_stride = qkv_row_stride;
  p.kpool = static_cast<const uint16_t*>(k_pool);
  p.vpool = static_cast<const uint16_t*>(v_pool);
  p.page_stride = pool_page_stride;
  p.page_table = page_table;
  p.ctx_lens = context_lens;
  p.blk_lens = block_lens;
  p.status = status_word;
  p.num_pages = num_pages;
  p.pt_stride = page_table_stride;
  p.R = num_requests;
  p.T = tokens_per_block;
  p.Hq = num_q_heads;
  p.Hkv = num_kv_heads;
  g_last_error.clear();
  hipLaunchKernelGGL(kv_append_kernel, dim3(num_requests, num_kv_heads), dim3(kApThreads), 0,
                     static_cast<hipStream_t>(stream), p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DA_ELAUNCH, std::string("launch failed: ") + hipGetErrorString(e));
  return DA_OK;
}

const char* drafter_attn_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
