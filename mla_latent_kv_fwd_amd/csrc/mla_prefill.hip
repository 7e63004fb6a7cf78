// mla_prefill.hip -- the expand path for one request's new tokens (declared in
// include/mla_prefill.h): expansion of cached latents into per-head keys and
// values, multi-head attention over one expanded chunk, and the LSE merge of
// the chunks.  ("MLA inference: two computation paths and FlashMLA", section
// "Two equivalent paths", path one; the same page's engine notes expand a long
// prefix in chunks and merge the chunks by LSE.)
//
// All contractions run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
//
// Expansion is a GEMM [tokens x 512] x [512 x (H x 256)] with the latent rows
// gathered through the block table: each workgroup keeps one head's weights of
// one product in registers and streams 64-token tiles of the latent through LDS
// with direct-to-LDS loads, two workgroups per CU (details at the kernel).
//
// Attention keeps the decode kernel's orientation -- scores as S^T = K . q^T,
// lane = query -- with 32 queries per wave, so every K or V^T fragment read
// from LDS feeds two MFMAs.  The rows of the two 16-token score tiles of a
// 32-token group are permuted (tile a: tokens 8(m/4) + m%4, tile b: + 4) so
// that a lane's eight probabilities are tokens 8g .. 8g+7 of the group: the
// B-operand of O^T += V^T . P^T with V^T read straight from a dims-major LDS
// tile.  Online softmax with the lazy rescale of the decode kernel.
#include <hip/hip_runtime.h>

#define MLA_HD __host__ __device__
#include "mla_launch.h"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))
// Read-only for the whole kernel: loads through it become scalar loads.
#define CONST_AS __attribute__((address_space(4)))

constexpr int kNope = 128, kRope = 64, kLat = 512, kDv = 128;
constexpr int kQK = kNope + kRope;   // 192
constexpr int kCacheRow = kLat + kRope;   // 576 numbers per cached token
constexpr int kPage = 64;
constexpr float kLazyRescale = 8.0f;      // log2 of the largest p kept unrescaled
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ bf16x8_t lds_b128(const char LDS_AS* p) { return *reinterpret_cast<const bf16x8_t LDS_AS*>(p); }

// The lane index, hidden from the optimiser: per-lane address terms derived from
// it are recomputed where they are used rather than kept live across loops.
__device__ __forceinline__ int opaque_lane() {
  int l = __lane_id();
  asm volatile("" : "+v"(l));
  return l;
}

__device__ __forceinline__ float row_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float row_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ===========================================================================
// Expansion
// ===========================================================================
// One GEMM per chunk: [tokens x 512] x [512 x (H x 256)], the latent rows
// gathered through the block table.  Each workgroup owns one column tile -- the
// 128 outputs of one head and one product (k^N with W_UK as C[n][t], v with W_UV
// as C[t][v]) -- and keeps that tile's weights in registers for the whole launch:
// four waves, each holding 32 weight rows x 512 latent columns as MFMA fragments
// (128 VGPRs).  The workgroup then streams its token tiles: stages of 64 latent
// rows x 128 columns (16 KiB) fill a three-stage LDS ring with direct-to-LDS
// loads, two stages in flight, one barrier per stage of 32 MFMAs per wave.  The
// latent is thus the only operand loaded per token tile: 64 KiB for 8.4 MFLOP
// (128 FLOP per byte, 32 B/clk per CU at the matrix pipe's full rate, under the
// ~54 B/clk a CU's direct-to-LDS loads sustain).  Wave w covers weight rows
// 32 w .. +32 and all 64 tokens of a tile.  A finished token tile is staged in
// LDS and leaves in whole rows with non-temporal stores issued at the next tile's
// first barrier; the k workgroups also copy the tile's RoPE keys, brought into LDS
// with direct-to-LDS loads along with the stages.  Two workgroups share each CU
// (74 KiB of LDS each, two waves per SIMD): a barrier holds only the four waves of
// one workgroup, and the other workgroup's waves keep the SIMD busy meanwhile.  A
// column tile's token tiles are split among 2 CUs / (2H) workgroups.
constexpr int kXThreads = 256;                 // four waves; two workgroups per CU
constexpr int kXWaves = kXThreads / 64;
constexpr int kXTok = 64;                      // tokens per token tile
constexpr int kXK = 128;                       // latent columns per stage
constexpr int kXStagesPerTile = kLat / kXK;    // 4
constexpr int kXBufs = 3;                      // ring depth
constexpr int kXStageBytes = kXTok * kXK * 2;  // 16 KiB
constexpr int kXLoads = kXStageBytes / 1024 / kXWaves;   // 4 one-KiB loads per wave per stage
constexpr int kXRopeBytes = kXTok * kRope * 2;           // 8 KiB of RoPE keys per token tile
constexpr int kXRopeLoads = kXRopeBytes / 1024 / kXWaves;   // 2 per wave
constexpr int kXRowPad = 272;                  // staged k rows (tokens): 256 bytes + 16
constexpr int kXVPad = kXTok * 2 + 16;         // staged v rows (dims): 128 bytes + 16
constexpr int kXStgBytes = kXTok * kXRowPad > 128 * kXVPad ? kXTok * kXRowPad : 128 * kXVPad;
constexpr int kXStgOff = kXBufs * kXStageBytes;
constexpr int kXRopeOff = kXStgOff + kXStgBytes;
constexpr int kXLdsBytes = kXRopeOff + kXRopeBytes;      // 74 KiB
static_assert(kXLoads * 1024 * kXWaves == kXStageBytes && kXRopeLoads * 1024 * kXWaves == kXRopeBytes, "");
static_assert(2 * kXLdsBytes <= 160 * 1024, "LDS of two workgroups per CU");

// Stage row r (one token, 256 bytes = 16 granules): granule j is stored at
// j ^ (r & 15), so the 16 rows of a fragment read (lane (g, q): granule 4 ks + g of
// row 16 i + q) fall in 16 different granule columns.  The fragment reads use the
// equivalent form (4 ks + g) ^ r = 4 (ks ^ (r >> 2)) + ((g ^ r) & 3).

// One 16-byte direct-to-LDS load per lane from a per-lane 64-bit address: lane i
// writes LDS[m0 + 16 i].  The wait states cover M0 written from a VALU-produced
// SGPR (as in the decode kernels' loads).
__device__ __forceinline__ void dma16_v(const void* gaddr, uint32_t lds_addr) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gaddr),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}

// s_waitcnt immediate for "vector memory counter <= n", other counters untouched.
#define XVMCNT(n) ((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4) | (15 << 8))

// Vector-memory operations this wave has issued after the loads of stage s + 1
// when it waits for them in the middle of iteration s (sl = s % 4, tile ti;
// valid while stage s + 2 exists).  Per wave, in issue order: the prologue's
// loads of stages 0-2 and, for k, the first tile's RoPE keys; in the middle of
// iteration s: at sl = 0 of a later tile the previous tile's output stores (four,
// six for k), at sl = 1 of a later tile (k) that tile's RoPE keys, then the loads
// of stage s + 3.
template <bool kIsK>
constexpr int x_younger(int sl, int ti) {
  const int rope = kIsK ? kXRopeLoads : 0;
  const int stores = kIsK ? 6 : 4;
  return kXLoads + (ti == 0 ? (sl <= 1 ? rope : 0) : (sl == 1 ? stores : 0) + (sl == 2 ? rope : 0));
}
// s_waitcnt takes an immediate: the counts above, spelled out (sl is a constant
// after unrolling; whether the tile is the first is a uniform scalar branch).
__device__ __forceinline__ void x_wait(int n) {
  switch (n) {
    case 4: __builtin_amdgcn_s_waitcnt(XVMCNT(4)); break;
    case 6: __builtin_amdgcn_s_waitcnt(XVMCNT(6)); break;
    case 8: __builtin_amdgcn_s_waitcnt(XVMCNT(8)); break;
    case 10: __builtin_amdgcn_s_waitcnt(XVMCNT(10)); break;
    case 12: __builtin_amdgcn_s_waitcnt(XVMCNT(12)); break;
    default: __builtin_amdgcn_s_waitcnt(XVMCNT(0)); break;
  }
}

template <bool kIsK>
__device__ __forceinline__ void expand_tiles(const uint16_t* __restrict__ cache, const int32_t* __restrict__ block_table,
                                             int t0, int ntok, int ld, int num_pages, const uint16_t* __restrict__ w,
                                             uint16_t* __restrict__ out, int h, int tt_begin, int tt_end,
                                             char* smem) {
  char LDS_AS* lds = (char LDS_AS*)smem;
  const uint32_t lds_addr = (uint32_t)(uintptr_t)smem;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int mo = 32 * wave;   // this wave's weight rows (outputs)
  const int tb = 0;           // every wave takes all 64 tokens of a tile

  // Weights: wf[m][k] = rows mo + 16 m + r of the head's 128, columns 32 k + 8 g .. +8.
  bf16x8_t wf[2][kLat / 32];
  {
    const uint16_t* wr = w + ((size_t)h * 128 + mo + r) * kLat + 8 * g;
#pragma unroll
    for (int m = 0; m < 2; m++)
#pragma unroll
      for (int k = 0; k < kLat / 32; k++)
        wf[m][k] = *reinterpret_cast<const bf16x8_t*>(wr + (size_t)16 * m * kLat + 32 * k);
  }
  __builtin_amdgcn_s_waitcnt(XVMCNT(0));   // the weights are in before the loads are counted by hand

  // Source rows of this lane's loads for one token tile, as cache row indices
  // (page * 64 + slot; the byte address is formed at each issue).  Stage load i
  // fills LDS block 8 i + wave: row 4 (8 i + wave) + lane / 16, physical granule
  // lane % 16, which holds logical granule (lane % 16) ^ (row & 15).  RoPE load i
  // fills block 8 i + wave of the RoPE area: token 8 (8 i + wave) + lane / 8,
  // granule lane % 8.  The tile's tokens lie on at most three pages, read through
  // the scalar cache.
  int ridx[kXLoads];
  int rridx[kXRopeLoads];
  auto set_rows = [&](int tt) {
    const int tile_t = tt * kXTok;
    const int pos_lo = t0 + tile_t;
    const int pos_hi = t0 + (tile_t + kXTok < ntok ? tile_t + kXTok : ntok) - 1;
    const int pg_lo = __builtin_amdgcn_readfirstlane(pos_lo / kPage);
    const int pg_hi = __builtin_amdgcn_readfirstlane(pos_hi / kPage);
    const int32_t CONST_AS* btc = (const int32_t CONST_AS*)block_table;
    auto page_at = [&](int u) {   // uniform: a scalar load
      const int pg = btc[pg_lo + u <= pg_hi ? pg_lo + u : pg_hi];
      return (pg < 0 || pg >= num_pages) ? 0 : pg;
    };
    const int p0 = page_at(0), p1 = page_at(1), p2 = page_at(2);
    auto row_index = [&](int row) {   // cache row of token tile_t + row (rows past the range repeat the last token)
      const int t = tile_t + row < ntok ? tile_t + row : ntok - 1;
      const int pos = t0 + t;
      const int d = pos / kPage - pg_lo;
      // Bit masks rather than a chain of selects, which the optimiser turns into a
      // lookup table in scratch memory.
      const int m0 = -(int)(d == 0), m1 = -(int)(d == 1);
      const int pg = (p0 & m0) | (p1 & m1) | (p2 & ~(m0 | m1));
      return pg * kPage + pos % kPage;
    };
    const int l = opaque_lane();
#pragma unroll
    for (int i = 0; i < kXLoads; i++) ridx[i] = row_index(4 * (kXWaves * i + wave) + (l >> 4));
    if (kIsK) {
#pragma unroll
      for (int i = 0; i < kXRopeLoads; i++) rridx[i] = row_index(8 * (kXWaves * i + wave) + (l >> 3));
    }
  };
  const char* cache_b = reinterpret_cast<const char*>(cache);
  auto issue = [&](int buf, int sl) {   // stage sl of the tile set_rows last took, into ring buffer buf
    const uint32_t base = lds_addr + buf * kXStageBytes;
    const int l = opaque_lane();
#pragma unroll
    for (int i = 0; i < kXLoads; i++) {
      const int row = 4 * (kXWaves * i + wave) + (l >> 4);
      const int gb = (((l & 15) ^ (row & 15)) << 4) + sl * kXK * 2;
      dma16_v(cache_b + (size_t)ridx[i] * (kCacheRow * 2) + gb, base + (kXWaves * i + wave) * 1024);
    }
  };
  auto issue_rope = [&]() {
    const int l = opaque_lane();
#pragma unroll
    for (int i = 0; i < kXRopeLoads; i++)
      dma16_v(cache_b + (size_t)rridx[i] * (kCacheRow * 2) + kLat * 2 + ((l & 7) << 4),
              lds_addr + kXRopeOff + (kXWaves * i + wave) * 1024);
  };

  f32x4_t acc[2][4];   // [weight-row tile][token tile] (k: C[n][t]; v: C[t][v] with the roles swapped)
#pragma unroll
  for (int m = 0; m < 2; m++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[m][j] = f32x4_t{};

  const int ntiles = tt_end - tt_begin;
  const int nst = ntiles * kXStagesPerTile;   // >= 4
  if (ntiles <= 0) return;
  // K-step ks of stage s, this wave's four token tiles: rows tb + 16 j + r, granule
  // 4 ks + g, stored at (4 ks + g) ^ r = 4 (ks ^ (r >> 2)) + ((g ^ r) & 3): a per-lane
  // offset per K-step, the tile j an immediate 4 KiB step.
  const int lrow = (tb + r) * (kXK * 2) + (((g ^ r) & 3) << 4);
  auto read_ks = [&](int s, int ks, bf16x8_t (&f)[4]) {
    const char LDS_AS* base = lds + (s % kXBufs) * kXStageBytes + lrow + ((ks ^ (r >> 2)) << 6);
#pragma unroll
    for (int j = 0; j < 4; j++) f[j] = lds_b128(base + j * 16 * (kXK * 2));
  };
  char LDS_AS* stg = lds + kXStgOff;
  // A finished tile: the accumulators into the LDS staging area (then cleared).
  auto stage_tile = [&](int tile_t) {
    // Lane (g, r) holds, for k, C[n = mo + 16 m + 4 g + e][t = tb + 16 j + r] and,
    // for v, C[t = tb + 16 j + 4 g + e][v = mo + 16 m + r].  The staged tile is bf16
    // rows: k rows are tokens (272 bytes: the head's 128 outputs + 16), v rows are
    // dims (144 bytes: the tile's 64 tokens + 16).  Tokens past the range are written
    // as zeros.  (The staging area was last read three barriers ago.)
#pragma unroll
    for (int m = 0; m < 2; m++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        bf16x4_t v4;
        if (kIsK) {
          const int tl = tb + 16 * j + r;
          const bool live = tile_t + tl < ntok;
#pragma unroll
          for (int e = 0; e < 4; e++) v4[e] = live ? (__bf16)acc[m][j][e] : (__bf16)0.f;
          *reinterpret_cast<bf16x4_t LDS_AS*>(stg + tl * kXRowPad + (mo + 16 * m + 4 * g) * 2) = v4;
        } else {
          const int tl = tb + 16 * j + 4 * g;
#pragma unroll
          for (int e = 0; e < 4; e++) v4[e] = tile_t + tl + e < ntok ? (__bf16)acc[m][j][e] : (__bf16)0.f;
          *reinterpret_cast<bf16x4_t LDS_AS*>(stg + (mo + 16 * m + r) * kXVPad + tl * 2) = v4;
        }
        acc[m][j] = f32x4_t{};
      }
  };
  // A staged tile leaves in whole rows: at the first barrier of the next tile,
  // under that stage's last MFMAs (every wave's staging writes precede the
  // barrier), or after the last tile.
  auto store_tile = [&](int tile_t) {
    // k: 64 rows x 16 granules, v: 128 rows x 8 granules; four per thread either way.
    // Non-temporal: the expanded chunk is far larger than the caches.
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int x = tid + u * kXThreads;
      if (kIsK) {
        const int gr = x & 15, row = x >> 4;
        const i32x4_t v = *reinterpret_cast<const i32x4_t LDS_AS*>(stg + row * kXRowPad + gr * 16);
        const int t = tile_t + row;
        if (t < ld) __builtin_nontemporal_store(v, reinterpret_cast<i32x4_t*>(out + ((size_t)h * ld + t) * kQK + 8 * gr));
      } else {
        const int gr = x & 7, row = x >> 3;
        const i32x4_t v = *reinterpret_cast<const i32x4_t LDS_AS*>(stg + row * kXVPad + gr * 16);
        const int t = tile_t + 8 * gr;   // ld is a multiple of 64: t < ld covers the granule
        if (t < ld) __builtin_nontemporal_store(v, reinterpret_cast<i32x4_t*>(out + ((size_t)h * kDv + row) * ld + t));
      }
    }
    if (kIsK) {
      // k^R: k[h][t][128 .. 191] = the cached RoPE key of token t (zeros past the range).
#pragma unroll
      for (int u = 0; u < 2; u++) {
        const int x = tid + u * kXThreads;
        const int part = x & 7, tok = x >> 3;
        const int t = tile_t + tok;
        i32x4_t v = *reinterpret_cast<const i32x4_t LDS_AS*>(lds + kXRopeOff + tok * (kRope * 2) + part * 16);
        if (t >= ntok) v = i32x4_t{};
        if (t < ld)
          __builtin_nontemporal_store(v, reinterpret_cast<i32x4_t*>(out + ((size_t)h * ld + t) * kQK + kNope + 8 * part));
      }
    }
  };
  set_rows(tt_begin);
  issue(0, 0);
  issue(1, 1);
  issue(2, 2);
  if (kIsK) issue_rope();
  x_wait(2 * kXLoads + (kIsK ? kXRopeLoads : 0));   // stage 0 has landed
  __syncthreads();
  bf16x8_t lf[4], ln[4];
  read_ks(0, 0, lf);
  for (int ti = 0; ti < ntiles; ti++) {
    const int tile_t = (tt_begin + ti) * kXTok;
#pragma unroll
    for (int sl = 0; sl < kXStagesPerTile; sl++) {
      const int s = ti * kXStagesPerTile + sl;
#pragma unroll
      for (int ks = 0; ks < kXK / 32; ks++) {
        if (ks + 1 < kXK / 32) {
          read_ks(s, ks + 1, ln);
        } else if (s + 1 < nst) {
          // Before the last K-step's MFMAs (the previous K-step's are still
          // running): stage s + 1 is in LDS for every wave and every wave is done
          // reading stage s, whose buffer takes stage s + 3.  Then the first
          // fragments of stage s + 1 are read under this K-step's MFMAs (after a
          // tile's last stage: after its epilogue, which needs the registers).
          if (s + 2 < nst) x_wait(x_younger<kIsK>(sl, ti > 0 ? 1 : 0));
          else __builtin_amdgcn_s_waitcnt(XVMCNT(0));
          __syncthreads();
          // The previous tile, staged before this barrier, leaves now; the next
          // barrier retires its reads of the staging and RoPE areas before this
          // tile's RoPE keys overwrite the latter.
          if (sl == 0 && ti > 0) store_tile(tile_t - kXTok);
          if (kIsK && sl == 1 && ti > 0) issue_rope();   // this tile's RoPE keys
          if (s + 3 < nst) {
            if (sl == 1) set_rows(tt_begin + ti + 1);   // stage s + 3 opens the next tile
            issue(s % kXBufs, (sl + 3) % kXStagesPerTile);
          }
          if (sl + 1 < kXStagesPerTile) read_ks(s + 1, 0, ln);
        }
        const int kg = sl * (kXK / 32) + ks;
#pragma unroll
        for (int m = 0; m < 2; m++)
#pragma unroll
          for (int j = 0; j < 4; j++)
            acc[m][j] = kIsK ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[m][kg], lf[j], acc[m][j], 0, 0, 0)
                             : __builtin_amdgcn_mfma_f32_16x16x32_bf16(lf[j], wf[m][kg], acc[m][j], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; j++) lf[j] = ln[j];
        __builtin_amdgcn_sched_barrier(0);   // keep the next K-step's reads ahead of these MFMAs
      }
    }

    stage_tile(tile_t);
    if (ti + 1 < ntiles) read_ks((ti + 1) * kXStagesPerTile, 0, lf);
  }
  __syncthreads();   // the last tile is staged
  store_tile((tt_end - 1) * kXTok);
}

// Workgroup i: column tile ct = i / nsp (ct < H: k^N of head ct; else v of head
// ct - H), token tiles [sp ntt / nsp, (sp + 1) ntt / nsp) with sp = i % nsp.
__global__ __launch_bounds__(kXThreads, 2) void mla_expand_kv_kernel(const uint16_t* __restrict__ cache,
                                                                    const int32_t* __restrict__ block_table, int t0,
                                                                    int ntok, int ld, int num_pages,
                                                                    const uint16_t* __restrict__ w_uk,
                                                                    const uint16_t* __restrict__ w_uv,
                                                                    uint16_t* __restrict__ k_out,
                                                                    uint16_t* __restrict__ vt_out, int H, int ntt,
                                                                    int nsp) {
  __shared__ __attribute__((aligned(1024))) char smem[kXLdsBytes];
  const int ct = blockIdx.x / nsp, sp = blockIdx.x % nsp;
  const int tt_begin = (int)((int64_t)sp * ntt / nsp), tt_end = (int)((int64_t)(sp + 1) * ntt / nsp);
  if (ct < H)
    expand_tiles<true>(cache, block_table, t0, ntok, ld, num_pages, w_uk, k_out, ct, tt_begin, tt_end, smem);
  else
    expand_tiles<false>(cache, block_table, t0, ntok, ld, num_pages, w_uv, vt_out, ct - H, tt_begin, tt_end, smem);
}

// ===========================================================================
// Attention over one expanded chunk
// ===========================================================================
constexpr int kAttThreads = 512;
constexpr int kAttWaves = kAttThreads / 64;
constexpr int kAttQ = 32 * kAttWaves;        // queries per workgroup (8 waves x 32)
constexpr int kAttBufs = 3;                  // LDS ring of key blocks, two in flight
constexpr int kKBlk = 64;                    // keys per LDS block
constexpr int kKBytes = kKBlk * kQK * 2;     // 24 KiB: 64 rows x 384 bytes
constexpr int kVBytes = kDv * kKBlk * 2;     // 16 KiB: 128 dim rows x 128 bytes
constexpr int kStage = kKBytes + kVBytes;    // 40 KiB
constexpr int kAttLoads = kStage / 1024 / kAttWaves;   // 5 one-KiB direct-to-LDS loads per wave per block
static_assert(kAttLoads * 1024 * kAttWaves == kStage && kKBytes % 1024 == 0, "whole one-KiB loads per wave");

// K rows (384 bytes, 24 granules): the low 3 bits of the granule index are XORed
// with bits (1, 3, 4) of the token, which makes the 16 (permuted) token rows of a
// score tile land in 16 bank groups.  V^T rows (128 bytes): granule ^ ((d >> 1) & 7).
__device__ __forceinline__ int k_off(int t, int j) {
  const int s = ((t >> 1) & 1) | ((t >> 2) & 6);
  return t * (kQK * 2) + (((j & ~7) | ((j & 7) ^ s)) << 4);
}
__device__ __forceinline__ int v_off(int d, int j) { return kKBytes + d * (kKBlk * 2) + ((j ^ ((d >> 1) & 7)) << 4); }

__global__ __launch_bounds__(kAttThreads, 1) void mla_prefill_attention_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kbuf, const uint16_t* __restrict__ vtbuf, int t0,
    int ntok, int ld, int n, int L, int H, float scale_log2, float* __restrict__ out, float* __restrict__ lse,
    uint16_t* __restrict__ out16) {
  __shared__ __attribute__((aligned(1024))) char smem[kAttBufs * kStage];
  char LDS_AS* lds = (char LDS_AS*)smem;
  const uint32_t lds_addr = (uint32_t)(uintptr_t)smem;
  // blockIdx -> (head, query block).  Workgroups are dealt to the 8 XCDs round robin
  // (linear id % 8); when H is a multiple of 8, head h runs only on XCD h % 8 with
  // all its query blocks together, so a head's K and V stay in that XCD's L2.
  // Causal rows late in the sequence see the most keys: they go first, the short
  // blocks fill the tail.
  const int nqb = gridDim.x;
  int h = blockIdx.y, qbi = blockIdx.x;
  if ((gridDim.y & 7) == 0) {
    const int lin = blockIdx.x + nqb * blockIdx.y;
    const int slot = lin >> 3, hh = slot / nqb;
    qbi = slot - hh * nqb;
    h = 8 * hh + (lin & 7);
  }
  const int qb = (nqb - 1 - qbi) * kAttQ;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;

  // Key blocks this workgroup needs: positions up to its last query's.
  const int qlast = min(qb + kAttQ - 1, n - 1);
  const int pos_first = L - n + qb;       // position of the first query of the block
  const int pos_last = L - n + qlast;
  const int nblk_all = ld / kKBlk;
  const int nblk = pos_last < t0 ? 0 : min(nblk_all, (pos_last - t0) / kKBlk + 1);

  // This wave's queries: tiles qt = 0, 1 of 16; lane r is query qw + 16 qt + r.
  const int qw = qb + 32 * wave;
  bf16x8_t qf[2][kQK / 32];
  int qpos[2];
#pragma unroll
  for (int qt = 0; qt < 2; qt++) {
    const int qi = qw + 16 * qt + r;
    const bool ok = qi < n;
    qpos[qt] = L - n + qi;
    const uint16_t* qrow = q + ((size_t)(ok ? qi : 0) * H + h) * kQK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kQK / 32; ks++) {
      const bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * ks);
      qf[qt][ks] = ok ? v : bf16x8_t{};
    }
  }

  // Key blocks stream HBM -> LDS with direct-to-LDS loads into a three-block ring.
  // One-KiB LDS block b of a ring slot (b < 24: K, else V^T) is loaded by wave
  // b % 8 as its load b / 8; lane l of it fills K granule gi = 64 b + l (row
  // t = gi / 24, physical granule gi % 24) or V^T granule x = 64 (b - 24) + l (row
  // d = x / 8, physical granule x % 8), so each lane reads the logical granule the
  // swizzle puts there.  Source offsets (elements, within the head's K or V^T) are
  // per lane and fixed; block kb adds kb * 64 rows of K or kb * 64 columns of V^T.
  const uint16_t* kh = kbuf + (size_t)h * ld * kQK;
  const uint16_t* vh = vtbuf + (size_t)h * kDv * ld;
  int soff[kAttLoads];
#pragma unroll
  for (int i = 0; i < kAttLoads; i++) {
    const int b = kAttWaves * i + wave;
    if (b < kKBytes / 1024) {
      const int gi = 64 * b + lane, t = gi / (kQK / 8), p = gi % (kQK / 8);
      const int sw = ((t >> 1) & 1) | ((t >> 2) & 6);
      const int j = (p & ~7) | ((p & 7) ^ sw);
      soff[i] = t * kQK + 8 * j;
    } else {
      const int x = 64 * (b - kKBytes / 1024) + lane, d = x >> 3, jp = x & 7;
      soff[i] = d * ld + 8 * (jp ^ ((d >> 1) & 7));
    }
  }
  auto issue = [&](int kb) {
    const uint32_t base = lds_addr + (kb % kAttBufs) * kStage;
#pragma unroll
    for (int i = 0; i < kAttLoads; i++) {
      const int b = kAttWaves * i + wave;
      const uint16_t* src = b < kKBytes / 1024 ? kh + (size_t)kb * kKBlk * kQK + soff[i] : vh + kb * kKBlk + soff[i];
      dma16_v(src, base + b * 1024);
    }
  };

  float m_ref[2] = {-INFINITY, -INFINITY};   // reference maximum (log2 units) per query tile
  float lsum[2] = {0.f, 0.f};
  f32x4_t o[2][kDv / 16];
#pragma unroll
  for (int qt = 0; qt < 2; qt++)
#pragma unroll
    for (int dt = 0; dt < kDv / 16; dt++) o[qt][dt] = f32x4_t{};

  // Score-tile row m of tile a is token 8(m/4) + m%4 of the 32-token group; tile b adds 4.
  const int ta = 8 * (r >> 2) + (r & 3);

  // The queries were loaded by the compiler; they are in before the loads are counted by hand.
  __builtin_amdgcn_s_waitcnt(XVMCNT(0));
  if (nblk > 0) issue(0);
  if (nblk > 1) issue(1);
  for (int kb = 0; kb < nblk; kb++) {
    // This wave's loads of block kb have landed (block kb + 1's may still be in flight).
    if (kb + 1 < nblk) __builtin_amdgcn_s_waitcnt(XVMCNT(kAttLoads));
    else __builtin_amdgcn_s_waitcnt(XVMCNT(0));
    __syncthreads();   // block kb is in LDS for every wave; slot (kb + 2) % 3 is free
    if (kb + 2 < nblk) issue(kb + 2);
    const char LDS_AS* base = lds + (kb % kAttBufs) * kStage;
    const int kpos0 = t0 + kb * kKBlk;   // position of the block's first key
    const bool need_mask = (kb * kKBlk + kKBlk > ntok) || (kpos0 + kKBlk - 1 > pos_first);
#pragma unroll
    for (int grp = 0; grp < 2; grp++) {
      f32x4_t s[2][2];   // [query tile][score tile a/b]
#pragma unroll
      for (int qt = 0; qt < 2; qt++) s[qt][0] = s[qt][1] = f32x4_t{};
      // K fragments read three K-steps ahead, pinned there (the compiler would
      // read them one or two K-steps ahead and wait on each pair).
      auto read_ka = [&](int ks) { return lds_b128(base + k_off(32 * grp + ta, 4 * ks + g)); };
      auto read_kb = [&](int ks) { return lds_b128(base + k_off(32 * grp + ta + 4, 4 * ks + g)); };
      bf16x8_t a0 = read_ka(0), b0 = read_kb(0), a1 = read_ka(1), b1 = read_kb(1);
      bf16x8_t a2 = read_ka(2), b2 = read_kb(2);
#pragma unroll
      for (int ks = 0; ks < kQK / 32; ks++) {
        bf16x8_t a3 = a2, b3 = b2;
        if (ks + 3 < kQK / 32) {
          a3 = read_ka(ks + 3);
          b3 = read_kb(ks + 3);
        }
#pragma unroll
        for (int qt = 0; qt < 2; qt++) {
          s[qt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[qt][ks], s[qt][0], 0, 0, 0);
          s[qt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0, qf[qt][ks], s[qt][1], 0, 0, 0);
        }
        a0 = a1;
        b0 = b1;
        a1 = a2;
        b1 = b2;
        a2 = a3;
        b2 = b3;
        __builtin_amdgcn_sched_barrier(0);
      }
      // s[qt][0][e] is token 32 grp + 8g + e, s[qt][1][e] token 32 grp + 8g + 4 + e.
      bf16x8_t pb[2];
#pragma unroll
      for (int qt = 0; qt < 2; qt++) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; e++) {
          x[e] = s[qt][0][e];
          x[4 + e] = s[qt][1][e];
        }
        if (need_mask) {
#pragma unroll
          for (int e = 0; e < 8; e++) {
            const int tl = kb * kKBlk + 32 * grp + 8 * g + e;   // key index within the chunk
            if (tl >= ntok || t0 + tl > qpos[qt]) x[e] = -INFINITY;
          }
        }
        float cmax = x[0];
#pragma unroll
        for (int e = 1; e < 8; e++) cmax = fmaxf(cmax, x[e]);
        cmax *= scale_log2;
        if (__builtin_amdgcn_ballot_w64(cmax > m_ref[qt] + kLazyRescale)) {
          const float rmax = row_max(cmax);
          const float m_new = rmax > m_ref[qt] + kLazyRescale ? rmax : m_ref[qt];
          const float alpha = m_ref[qt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref[qt] - m_new);
          lsum[qt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < kDv / 16; dt++) o[qt][dt] *= alpha;
          m_ref[qt] = m_new;
        }
        const float mu = m_ref[qt] == -INFINITY ? 0.f : m_ref[qt];
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], scale_log2, -mu));
          lsum[qt] += p;
          pb[qt][e] = (__bf16)p;
        }
      }
      // O^T[d][query] += V^T[d][token] . P^T[token][query]: A = 16 dims x 32 tokens of V^T.
      // V^T fragments read three dim tiles ahead, pinned there: otherwise the
      // compiler reads each right before its MFMAs and every pair waits a full LDS
      // latency.
      auto read_vf = [&](int dt) { return lds_b128(base + v_off(16 * dt + r, 4 * grp + g)); };
      bf16x8_t v0 = read_vf(0), v1 = read_vf(1), v2 = read_vf(2);
#pragma unroll
      for (int dt = 0; dt < kDv / 16; dt++) {
        bf16x8_t v3 = v2;
        if (dt + 3 < kDv / 16) v3 = read_vf(dt + 3);
#pragma unroll
        for (int qt = 0; qt < 2; qt++) o[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v0, pb[qt], o[qt][dt], 0, 0, 0);
        v0 = v1;
        v1 = v2;
        v2 = v3;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // Finalise: lane (g, r) holds O^T[16 dt + 4g + e][query qw + 16 qt + r].  The
  // normalised rows go out in fp32 (a chunk's part, merged later), or, when the
  // chunk is the whole context, in bf16 as the final output (the merge of a single
  // part would round the same fp32 numbers the same way).
#pragma unroll
  for (int qt = 0; qt < 2; qt++) {
    const float ltot = row_sum(lsum[qt]);
    const int qi = qw + 16 * qt + r;
    if (qi >= n) continue;
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    if (out16) {   // uniform
      uint16_t* orow = out16 + ((size_t)qi * H + h) * kDv + 4 * g;
#pragma unroll
      for (int dt = 0; dt < kDv / 16; dt++) {
        const f32x4_t x = o[qt][dt] * inv;
        bf16x4_t w;
#pragma unroll
        for (int e = 0; e < 4; e++) w[e] = (__bf16)x[e];
        *reinterpret_cast<bf16x4_t*>(orow + 16 * dt) = w;
      }
    } else {
      float* orow = out + ((size_t)qi * H + h) * kDv + 4 * g;
#pragma unroll
      for (int dt = 0; dt < kDv / 16; dt++) *reinterpret_cast<f32x4_t*>(orow + 16 * dt) = o[qt][dt] * inv;
    }
    if (g == 0) lse[(size_t)qi * H + h] = ltot > 0.f ? (m_ref[qt] + __builtin_amdgcn_logf(ltot)) * kLn2 : -INFINITY;
  }
}

// ===========================================================================
// LSE merge of J partials
// ===========================================================================
constexpr int kMrgThreads = 256;
constexpr int kMrgRows = kMrgThreads / (kDv / 8);   // 16 rows per workgroup, 8 columns per thread

__global__ __launch_bounds__(kMrgThreads) void mla_lse_merge_kernel(int rows, int J, const float* __restrict__ parts,
                                                                   const float* __restrict__ lparts,
                                                                   uint16_t* __restrict__ out, float* __restrict__ lse) {
  const int row = blockIdx.x * kMrgRows + threadIdx.x / (kDv / 8);
  const int col = (threadIdx.x % (kDv / 8)) * 8;
  if (row >= rows) return;
  float m = -INFINITY, z = 0.f;
  f32x4_t a0 = f32x4_t{}, a1 = f32x4_t{};
  for (int j = 0; j < J; j++) {
    const float lj = lparts[(size_t)j * rows + row];
    if (lj == -INFINITY) continue;   // no weight; its row is not read
    const f32x4_t* src = reinterpret_cast<const f32x4_t*>(parts + ((size_t)j * rows + row) * kDv + col);
    const float m2 = fmaxf(m, lj);
    const float keep = __expf(m - m2);
    const float w = __expf(lj - m2);
    z = z * keep + w;
    a0 = a0 * keep + w * src[0];
    a1 = a1 * keep + w * src[1];
    m = m2;
  }
  const float inv = z > 0.f ? 1.f / z : 0.f;
  bf16x8_t res;
#pragma unroll
  for (int e = 0; e < 4; e++) {
    res[e] = (__bf16)(a0[e] * inv);
    res[4 + e] = (__bf16)(a1[e] * inv);
  }
  *reinterpret_cast<bf16x8_t*>(out + (size_t)row * kDv + col) = res;
  if (col == 0) lse[row] = z > 0.f ? m + __logf(z) : -INFINITY;
}

}  // namespace

hipError_t launch_expand_kv(const uint16_t* cache, const int32_t* block_table, int t0, int ntok, int num_pages,
                            const uint16_t* w_uk, const uint16_t* w_uv, uint16_t* k_out, uint16_t* vt_out, int H,
                            hipStream_t stream) {
  int ld = (ntok + 63) / 64 * 64;
  int ntt = (ld + kXTok - 1) / kXTok;
  const int nct = 2 * H;
  // Two workgroups per CU: a column tile's token tiles are split among 2 cus / nct workgroups.
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  int nsp = 2 * cus / nct > 1 ? 2 * cus / nct : 1;
  nsp = nsp < ntt ? nsp : ntt;
  void* args[] = {(void*)&cache, (void*)&block_table, (void*)&t0,    (void*)&ntok,   (void*)&ld, (void*)&num_pages,
                  (void*)&w_uk,  (void*)&w_uv,        (void*)&k_out, (void*)&vt_out, (void*)&H,  (void*)&ntt,
                  (void*)&nsp};
  return hipLaunchKernel((const void*)mla_expand_kv_kernel, dim3(nct * nsp), dim3(kXThreads), args, 0, stream);
}

hipError_t launch_prefill_attention(const uint16_t* q, const uint16_t* k, const uint16_t* vt, int t0, int ntok, int n,
                                    int L, int H, float softmax_scale, float* out, float* lse, uint16_t* out16,
                                    hipStream_t stream) {
  int ld = (ntok + 63) / 64 * 64;
  float scale_log2 = softmax_scale * 1.4426950408889634f;
  void* args[] = {(void*)&q, (void*)&k, (void*)&vt, (void*)&t0, (void*)&ntok, (void*)&ld, (void*)&n,
                  (void*)&L, (void*)&H, (void*)&scale_log2, (void*)&out, (void*)&lse, (void*)&out16};
  return hipLaunchKernel((const void*)mla_prefill_attention_kernel, dim3((n + kAttQ - 1) / kAttQ, H),
                         dim3(kAttThreads), args, 0, stream);
}

hipError_t launch_lse_merge(int rows, int J, const float* parts, const float* lparts, uint16_t* out, float* lse,
                            hipStream_t stream) {
  void* args[] = {(void*)&rows, (void*)&J, (void*)&parts, (void*)&lparts, (void*)&out, (void*)&lse};
  return hipLaunchKernel((const void*)mla_lse_merge_kernel, dim3((rows + kMrgRows - 1) / kMrgRows),
                         dim3(kMrgThreads), args, 0, stream);
}

}  // namespace mla
