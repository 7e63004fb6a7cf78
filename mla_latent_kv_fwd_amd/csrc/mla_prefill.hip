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
// gathered through the block table: 128-token by two-head tiles streamed through
// LDS with direct-to-LDS loads, two workgroups per CU (details at the kernel).
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
__device__ __forceinline__ void lds_w128(char LDS_AS* p, bf16x8_t v) { *reinterpret_cast<bf16x8_t LDS_AS*>(p) = v; }

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
// One GEMM per chunk: [tokens x 512] x [512 x (H x 256)].  A workgroup of four
// waves owns a macro tile of 128 tokens by two heads' 128 outputs of one product
// (256 weight rows), and each wave a 128 x 64 part of it, so a fragment read from
// LDS feeds four or eight MFMAs.  The two operand tiles (32 latent columns of
// 128 token rows and 256 weight rows per stage, 24 KiB) stream HBM -> LDS with
// direct-to-LDS loads into a ring of three stages, two in flight; one barrier
// per stage of 32 MFMAs per wave.  Two workgroups share a compute unit and cover
// each other's load latency and epilogue.  The latent rows are gathered through
// the block table when the per-lane row addresses are set up; rows past the
// range repeat the last token and their outputs are written as zeros.  The
// output tile is staged in LDS and leaves in whole rows with non-temporal stores.
constexpr int kXTok = 128;                     // tokens per macro tile
constexpr int kXW = 256;                       // weight rows per macro tile (two heads)
constexpr int kXK = 32;                        // latent columns per stage
constexpr int kXStages = kLat / kXK;           // 16
constexpr int kXBufs = 3;                      // ring depth
constexpr int kXThreads = 256;                 // four waves
constexpr int kXBufBytes = (kXTok + kXW) * kXK * 2;   // 24 KiB
constexpr int kXLoads = kXBufBytes / 1024 / (kXThreads / 64);   // 6 one-KiB loads per wave per stage
static_assert(kXLoads * 1024 * (kXThreads / 64) == kXBufBytes, "");
static_assert(2 * 128 * 272 <= kXBufs * kXBufBytes, "the staged output tile fits in the ring");
// Operand row r of a stage (64 bytes): granule j stored at j ^ xp_swz(r).  The
// fragment read (lane (g, q): granule g of row 16 i + q) runs at the LDS's full
// rate with this map; the map j ^ ((r >> 2) & 3), which spreads 16 rows over 16
// 16-byte bank groups, ran at 57% of it (timed over all 256 linear maps of the
// row's low 4 bits to 2 bits; several reach the full rate).
__device__ __forceinline__ int xp_swz(int r) { return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 2)) & 1) << 1); }
__device__ __forceinline__ int xp_off(int r, int j) { return r * 64 + ((j ^ xp_swz(r)) << 4); }

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

// Workgroup (token tile tt, column tile ct): ct < HP forms k^N of heads 2ct, 2ct + 1
// as C[n][t] (A = W_UK rows, B = latent rows); ct >= HP forms v of heads
// 2(ct - HP), +1 as C[t][v] (A = latent rows, B = W_UV rows).  HP = ceil(H / 2).
// A stage holds the A tile first, then the B tile.
__global__ __launch_bounds__(kXThreads, 2) void mla_expand_kv_kernel(const uint16_t* __restrict__ cache,
                                                                    const int32_t* __restrict__ block_table, int t0,
                                                                    int ntok, int ld, int num_pages,
                                                                    const uint16_t* __restrict__ w_uk,
                                                                    const uint16_t* __restrict__ w_uv,
                                                                    uint16_t* __restrict__ k_out,
                                                                    uint16_t* __restrict__ vt_out, int H, int ntt) {
  __shared__ __attribute__((aligned(1024))) char smem[kXBufs * kXBufBytes];
  char LDS_AS* lds = (char LDS_AS*)smem;
  const uint32_t lds_addr = (uint32_t)(uintptr_t)smem;
  const int HP = (H + 1) / 2;
  // blockIdx -> tiles.  Workgroups are dealt to the 8 XCDs round robin; when the
  // counts allow, XCD x gets token tiles [x ntt/8, (x+1) ntt/8) of every column
  // tile, column tiles outermost, so its L2 holds those latent rows for the whole
  // launch and the weight tiles of the column tiles in progress.
  int tt, ct;
  {
    const int nblk = gridDim.x;
    const int lin = blockIdx.x;
    if ((ntt & 7) == 0 && (nblk & 7) == 0) {
      const int per = ntt >> 3, idx = lin >> 3;
      tt = (lin & 7) * per + idx % per;
      ct = idx / per;
    } else {
      tt = lin % ntt;
      ct = lin / ntt;
    }
  }
  const bool is_k = ct < HP;
  const int hp = is_k ? ct : ct - HP;
  const int tile_t = tt * kXTok;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  // 1-KiB blocks of a stage: k: weights 0..15, latent 16..23; v: latent 0..7, weights 8..23.
  const int lat_blk0 = is_k ? kXW / 16 : 0;
  const int w_blk0 = is_k ? 0 : kXTok / 16;

  // Per-lane source rows of this wave's six loads of a stage: load i is block
  // b = 4 i + wave; lane granule G = 64 (b - first block of its tile) + lane is
  // row G / 4 of that tile, stored granule G % 4, which holds logical granule
  // (G % 4) ^ xp_swz(row).
  const uint16_t* wt = (is_k ? w_uk : w_uv);
  // The tile's tokens lie on at most three pages: their block-table entries are
  // read once through the scalar cache (uniform loads), not once per lane.
  const int pos_lo = t0 + tile_t;
  const int pos_hi = t0 + (tile_t + kXTok - 1 < ntok - 1 ? tile_t + kXTok - 1 : ntok - 1);
  const int pg_lo = __builtin_amdgcn_readfirstlane(pos_lo / kPage);
  const int pg_hi = __builtin_amdgcn_readfirstlane(pos_hi / kPage);
  const int32_t CONST_AS* btc = (const int32_t CONST_AS*)block_table;
  int pages3[3];
#pragma unroll
  for (int u = 0; u < 3; u++) {
    int pg = btc[pg_lo + u <= pg_hi ? pg_lo + u : pg_hi];
    pages3[u] = (pg < 0 || pg >= num_pages) ? 0 : pg;
  }
  auto page_of = [&](int pos) {   // pos within [pos_lo, pos_hi]
    const int d = pos / kPage - pg_lo;
    return d == 0 ? pages3[0] : (d == 1 ? pages3[1] : pages3[2]);
  };
  const char* src[kXLoads];
#pragma unroll
  for (int i = 0; i < kXLoads; i++) {
    const int b = 4 * i + wave;
    const bool latent = is_k ? b >= lat_blk0 : b < w_blk0;
    const int G = 64 * (b - (latent ? lat_blk0 : w_blk0)) + lane;
    const int row = G >> 2;
    const int j = (G & 3) ^ xp_swz(row);
    const uint16_t* p;
    if (latent) {
      int t = tile_t + row;
      t = t < ntok ? t : ntok - 1;
      const int pos = t0 + t;
      p = cache + ((size_t)page_of(pos) * kPage + pos % kPage) * kCacheRow;
    } else {
      int h = 2 * hp + (row >> 7);
      h = h < H ? h : H - 1;
      p = wt + ((size_t)h * kNope + (row & 127)) * kLat;
    }
    src[i] = reinterpret_cast<const char*>(p) + 16 * j;
  }
  __builtin_amdgcn_s_waitcnt(XVMCNT(0));   // block-table reads done before the loads are counted by hand

  auto issue = [&](int st) {
    const uint32_t base = lds_addr + (st % kXBufs) * kXBufBytes;
#pragma unroll
    for (int i = 0; i < kXLoads; i++) dma16_v(src[i] + st * kXK * 2, base + (4 * i + wave) * 1024);
  };

  // This wave's part: A rows abase + 16 i + r (i < 8), B rows bbase + 16 j + r (j < 4).
  const int abase = is_k ? 128 * (wave & 1) : 0;
  const int bbase = is_k ? 64 * (wave >> 1) : 64 * wave;
  const int b_off = (is_k ? kXW : kXTok) * kXK * 2;   // the B tile's byte offset in a stage
  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = f32x4_t{};

  issue(0);
  issue(1);
  for (int st = 0; st < kXStages; st++) {
    if (st + 1 < kXStages) __builtin_amdgcn_s_waitcnt(XVMCNT(kXLoads));   // stage st + 1 may stay in flight
    else __builtin_amdgcn_s_waitcnt(XVMCNT(0));
    __syncthreads();   // every wave's loads of stage st have landed; buffer (st - 1) % 3 is free
    if (st + 2 < kXStages) issue(st + 2);
    const char LDS_AS* base = lds + (st % kXBufs) * kXBufBytes;
    bf16x8_t af[8], bfr[4];
#pragma unroll
    for (int i = 0; i < 8; i++) af[i] = lds_b128(base + xp_off(abase + 16 * i + r, g));
#pragma unroll
    for (int j = 0; j < 4; j++) bfr[j] = lds_b128(base + b_off + xp_off(bbase + 16 * j + r, g));
#pragma unroll
    for (int i = 0; i < 8; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
  }

  // Epilogue through LDS, so that global stores are whole 256-byte rows: lane (g, r)
  // holds C[abase + 16 i + 4 g + e][bbase + 16 j + r], e = 0..3.  The staged tile
  // is [head][row][128 values] in bf16 with rows padded to 272 bytes (16 lanes of
  // a store land in 16 bank groups): k^N rows are tokens (values = the head's 128
  // outputs), v rows are the head's 128 dims (values = the tile's 128 tokens).
  // Tokens past the range are written as zeros.
  constexpr int kRowPad = 272;
  __syncthreads();   // every wave is done with the ring
  char LDS_AS* stg = lds;
  if (is_k) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int tl = bbase + 16 * j + r;   // token within the tile
      const bool live = tile_t + tl < ntok;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int m = abase + 16 * i + 4 * g;
        bf16x4_t w;
#pragma unroll
        for (int e = 0; e < 4; e++) w[e] = live ? (__bf16)acc[i][j][e] : (__bf16)0.f;
        *reinterpret_cast<bf16x4_t LDS_AS*>(stg + ((m >> 7) * kXTok + tl) * kRowPad + (m & 127) * 2) = w;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int tl = 16 * i + 4 * g;   // first of four tokens within the tile
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int n = bbase + 16 * j + r;
        bf16x4_t w;
#pragma unroll
        for (int e = 0; e < 4; e++) w[e] = tile_t + tl + e < ntok ? (__bf16)acc[i][j][e] : (__bf16)0.f;
        *reinterpret_cast<bf16x4_t LDS_AS*>(stg + ((n >> 7) * kDv + (n & 127)) * kRowPad + tl * 2) = w;
      }
    }
  }
  __syncthreads();
  // 2 heads x 128 rows x 16 granules: 16 per thread, 16 consecutive lanes per row.
#pragma unroll 4
  for (int x = tid; x < 2 * 128 * 16; x += kXThreads) {
    const int gr = x & 15, row = (x >> 4) & 127, hh = x >> 11;
    const int h = 2 * hp + hh;
    if (h >= H) continue;
    const bf16x8_t v = *reinterpret_cast<const bf16x8_t LDS_AS*>(stg + (hh * 128 + row) * kRowPad + gr * 16);
    // Non-temporal: the expanded chunk is far larger than the caches (measured: the
    // kernel 21% faster than with ordinary stores).
    const i32x4_t vi = __builtin_bit_cast(i32x4_t, v);
    if (is_k) {
      const int t = tile_t + row;
      if (t < ld) __builtin_nontemporal_store(vi, reinterpret_cast<i32x4_t*>(k_out + ((size_t)h * ld + t) * kQK + 8 * gr));
    } else {
      const int t = tile_t + 8 * gr;   // ld is a multiple of 64: t < ld covers the granule
      if (t < ld) __builtin_nontemporal_store(vi, reinterpret_cast<i32x4_t*>(vt_out + ((size_t)h * kDv + row) * ld + t));
    }
  }
  if (is_k) {
    // k^R: k[h][t][128 .. 191] = the cached RoPE key of token t (zeros past the range).
    for (int x = tid; x < kXTok * 2 * (kRope / 8); x += kXThreads) {
      const int part = x & 7, hh = (x >> 3) & 1, jt = x >> 4;
      const int t = tile_t + jt, h = 2 * hp + hh;
      if (t >= ld || h >= H) continue;
      bf16x8_t v = bf16x8_t{};
      if (t < ntok) {
        const int pos = t0 + t;
        v = *reinterpret_cast<const bf16x8_t*>(cache + ((size_t)page_of(pos) * kPage + pos % kPage) * kCacheRow + kLat +
                                                8 * part);
      }
      __builtin_nontemporal_store(__builtin_bit_cast(i32x4_t, v),
                                  reinterpret_cast<i32x4_t*>(k_out + ((size_t)h * ld + t) * kQK + kNope + 8 * part));
    }
  }
}

// ===========================================================================
// Attention over one expanded chunk
// ===========================================================================
constexpr int kAttThreads = 256;
constexpr int kAttQ = 128;                   // queries per workgroup (4 waves x 32)
constexpr int kKBlk = 64;                    // keys per LDS block
constexpr int kKBytes = kKBlk * kQK * 2;     // 24 KiB: 64 rows x 384 bytes
constexpr int kVBytes = kDv * kKBlk * 2;     // 16 KiB: 128 dim rows x 128 bytes
constexpr int kStage = kKBytes + kVBytes;    // 40 KiB
constexpr int kGranK = kKBlk * (kQK / 8);    // 1,536 granules
constexpr int kGranV = kDv * (kKBlk / 8);    // 1,024 granules
static_assert(kGranK % kAttThreads == 0 && kGranV % kAttThreads == 0, "whole granules per thread");

// K rows (384 bytes, 24 granules): the low 3 bits of the granule index are XORed
// with bits (1, 3, 4) of the token, which makes the 16 (permuted) token rows of a
// score tile land in 16 bank groups.  V^T rows (128 bytes): granule ^ ((d >> 1) & 7).
__device__ __forceinline__ int k_off(int t, int j) {
  const int s = ((t >> 1) & 1) | ((t >> 2) & 6);
  return t * (kQK * 2) + (((j & ~7) | ((j & 7) ^ s)) << 4);
}
__device__ __forceinline__ int v_off(int d, int j) { return kKBytes + d * (kKBlk * 2) + ((j ^ ((d >> 1) & 7)) << 4); }

__global__ __launch_bounds__(kAttThreads, 2) void mla_prefill_attention_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kbuf, const uint16_t* __restrict__ vtbuf, int t0,
    int ntok, int ld, int n, int L, int H, float scale_log2, float* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kStage];
  char LDS_AS* lds = (char LDS_AS*)smem;
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
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

  // Block loads: K granules gi = tid + 256 u (u < 6), V^T granules x = tid + 256 u (u < 4).
  const uint16_t* kh = kbuf + (size_t)h * ld * kQK;
  const uint16_t* vh = vtbuf + (size_t)h * kDv * ld;
  constexpr int kUK = kGranK / kAttThreads, kUV = kGranV / kAttThreads;   // 6, 4
  bf16x8_t pre[kUK + kUV];
  auto fetch = [&](int kb) {
#pragma unroll
    for (int u = 0; u < kUK; u++) {
      const int gi = tid + u * kAttThreads;
      const int t = gi / (kQK / 8), j = gi % (kQK / 8);
      pre[u] = *reinterpret_cast<const bf16x8_t*>(kh + (size_t)(kb * kKBlk + t) * kQK + 8 * j);
    }
#pragma unroll
    for (int u = 0; u < kUV; u++) {
      const int x = tid + u * kAttThreads, d = x >> 3, j = x & 7;
      pre[kUK + u] = *reinterpret_cast<const bf16x8_t*>(vh + (size_t)d * ld + kb * kKBlk + 8 * j);
    }
  };
  auto stash = [&](int buf) {
    char LDS_AS* base = lds + buf * kStage;
#pragma unroll
    for (int u = 0; u < kUK; u++) {
      const int gi = tid + u * kAttThreads;
      lds_w128(base + k_off(gi / (kQK / 8), gi % (kQK / 8)), pre[u]);
    }
#pragma unroll
    for (int u = 0; u < kUV; u++) {
      const int x = tid + u * kAttThreads;
      lds_w128(base + v_off(x >> 3, x & 7), pre[kUK + u]);
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

  if (nblk > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();
  for (int kb = 0; kb < nblk; kb++) {
    if (kb + 1 < nblk) fetch(kb + 1);
    const char LDS_AS* base = lds + (kb & 1) * kStage;
    const int kpos0 = t0 + kb * kKBlk;   // position of the block's first key
    const bool need_mask = (kb * kKBlk + kKBlk > ntok) || (kpos0 + kKBlk - 1 > pos_first);
#pragma unroll
    for (int grp = 0; grp < 2; grp++) {
      f32x4_t s[2][2];   // [query tile][score tile a/b]
#pragma unroll
      for (int qt = 0; qt < 2; qt++) s[qt][0] = s[qt][1] = f32x4_t{};
#pragma unroll
      for (int ks = 0; ks < kQK / 32; ks++) {
        const bf16x8_t ka = lds_b128(base + k_off(32 * grp + ta, 4 * ks + g));
        const bf16x8_t kbf = lds_b128(base + k_off(32 * grp + ta + 4, 4 * ks + g));
#pragma unroll
        for (int qt = 0; qt < 2; qt++) {
          s[qt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[qt][ks], s[qt][0], 0, 0, 0);
          s[qt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kbf, qf[qt][ks], s[qt][1], 0, 0, 0);
        }
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
#pragma unroll
      for (int dt = 0; dt < kDv / 16; dt++) {
        const bf16x8_t vf = lds_b128(base + v_off(16 * dt + r, 4 * grp + g));
#pragma unroll
        for (int qt = 0; qt < 2; qt++) o[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[qt], o[qt][dt], 0, 0, 0);
      }
    }
    if (kb + 1 < nblk) stash((kb + 1) & 1);   // that buffer was last read in block kb-1
    __syncthreads();
  }

  // Finalise: lane (g, r) holds O^T[16 dt + 4g + e][query qw + 16 qt + r].
#pragma unroll
  for (int qt = 0; qt < 2; qt++) {
    const float ltot = row_sum(lsum[qt]);
    const int qi = qw + 16 * qt + r;
    if (qi >= n) continue;
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    float* orow = out + ((size_t)qi * H + h) * kDv + 4 * g;
#pragma unroll
    for (int dt = 0; dt < kDv / 16; dt++) *reinterpret_cast<f32x4_t*>(orow + 16 * dt) = o[qt][dt] * inv;
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
  const int nct = 2 * ((H + 1) / 2);
  void* args[] = {(void*)&cache, (void*)&block_table, (void*)&t0,    (void*)&ntok,   (void*)&ld, (void*)&num_pages,
                  (void*)&w_uk,  (void*)&w_uv,        (void*)&k_out, (void*)&vt_out, (void*)&H,  (void*)&ntt};
  return hipLaunchKernel((const void*)mla_expand_kv_kernel, dim3(ntt * nct), dim3(kXThreads), args, 0, stream);
}

hipError_t launch_prefill_attention(const uint16_t* q, const uint16_t* k, const uint16_t* vt, int t0, int ntok, int n,
                                    int L, int H, float softmax_scale, float* out, float* lse, hipStream_t stream) {
  int ld = (ntok + 63) / 64 * 64;
  float scale_log2 = softmax_scale * 1.4426950408889634f;
  void* args[] = {(void*)&q, (void*)&k, (void*)&vt, (void*)&t0, (void*)&ntok, (void*)&ld, (void*)&n,
                  (void*)&L, (void*)&H, (void*)&scale_log2, (void*)&out, (void*)&lse};
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
