// mla_decode_kernel.hip -- MLA absorb-path decode over a paged latent cache on
// gfx950 (MI355X).
//
// What it computes, per query row r of request b and the cached tokens t the row
// may see: s_t = scale * q~_r . [c_t ; k^R_t] (one 576-wide dot product: latent
// part plus RoPE part), softmax over t, out_r = sum_t p_t c_t (the 512-wide
// latent is the value), lse_r = ln sum_t exp(s_t).  ("MLA inference: two
// computation paths and FlashMLA", section "Two equivalent paths": score
// equation and path two; FlashMLA guide, Architecture step 3: the two score
// parts summed and scaled by 1/sqrt(192); step 4: online softmax.)
//
// How it maps onto CDNA4.  A persistent workgroup of 8 waves owns up to 128
// query rows (heads x new tokens) of one request and walks its stretch of
// pages (the split plan).  All 128 rows share each cached token, so one token
// read from HBM feeds 128 rows: the handbook's "Decode attention becomes a
// compute problem" section -- heads as the M dimension, the latent as K, one
// block handling all heads and a stretch of KV.
//   * Pages stream HBM -> LDS with direct-to-LDS loads (no VGPR staging) into a
//     ring of 4 slots of 32 tokens (4 x 36 KiB), three slots in flight.  A
//     chunk's page comes from a block-table window held one entry per lane
//     (a readlane, no scalar load to wait on).  Waves 0-3 issue all of a
//     chunk's loads, nine each, from one asm block with precomputed per-lane
//     offsets; waves 4-7, which set the pace, issue none.
//   * Each wave holds its 16 rows of q~ in registers (18 MFMA B-fragments) and
//     computes S^T = KV . q~^T with v_mfma_f32_16x16x32_bf16: tokens are M and
//     rows are N, so every lane owns one row and the softmax statistics need two
//     cross-lane swaps (the four 16-lane groups share a row).
//   * O^T = V^T . P^T on the same MFMA: V^T fragments come straight from the
//     token-major LDS slot through the gfx950 transposing LDS read, P^T is the
//     score accumulator converted to bf16 in place, and O^T keeps lane = row,
//     so the softmax rescale is a per-lane scalar.  Two waves share each SIMD,
//     so one wave's softmax overlaps the other's MFMAs, and each wave fits in
//     256 registers (q~ 72, O 128, scores 8, the rest working set).
//   * The running maximum is rescaled lazily: O and the normaliser are only
//     rescaled when a new maximum exceeds the reference by more than 2^8.  The
//     test is on each lane's own maximum (one ballot); the cross-lane row
//     maximum is formed only when it fires.  The scale is folded into the
//     exponent's FMA.
//   * The LDS reads of the two contractions are pinned two K-steps (scores) and
//     three dim tiles (values) ahead with scheduling barriers: without them the
//     compiler sinks each read to its use and every MFMA waits a full LDS
//     latency.  The registers for that depth come from rebuilding the loading
//     waves' per-lane load offsets at each issue instead of keeping them live.
//   * Tokens past the request's length are never loaded (their rows are
//     replaced by the last valid token) and are masked to -inf, so stale or NaN
//     bytes in a partly used last page cannot reach the output.
#include <hip/hip_runtime.h>

#define MLA_HD __host__ __device__
#include "mla_decode.h"
#include "mla_launch.h"
#include "mla_workspace.h"

namespace mla {
namespace {

#include "mla_decode_common.h"


constexpr int kChunk = 32;                         // tokens per LDS slot
constexpr int kSlots = 4;                          // ring depth
constexpr int kRowBytes = kHeadDimQK * 2;          // 1152 bytes per bf16 token row
constexpr int kGranPerRow = kRowBytes / 16;        // 72 16-byte granules
constexpr int kSlotBytes = kChunk * kRowBytes;     // 36864
constexpr int kSlotBlocks = kSlotBytes / 1024;     // 36 blocks of 64 granules (one wave-wide load each)
constexpr int kKSteps = kHeadDimQK / 32;           // 18 MFMA K-steps for QK

static_assert(kSlots * kSlotBytes <= 160 * 1024, "LDS ring must fit in 160 KiB");


// XOR swizzle of the low 3 bits of a row's 16-byte granule index by bits 1-2
// of the token index.  Picked by timing every linear 4->3 bit swizzle on both
// read patterns (a 16-token b128 QK read, an 8-token transposing PV read): this
// one runs both at the LDS's linear-access rate.
__device__ __forceinline__ int swz(int tok) { return tok & 6; }


// A slot is 36 one-KiB direct-to-LDS loads, all issued by waves 0-3 (nine
// each).  On each SIMD the older wave (0-3) wins issue arbitration and then
// waits at the chunk barrier for its sibling (4-7), so the load issue -- which
// stalls while the CU's address unit drains the burst -- is moved off the
// waves that set the pace.
constexpr int kLoadWaves = 4;
constexpr int kLoadsPerWave = kSlotBlocks / kLoadWaves;   // 9
static_assert(kLoadsPerWave * kLoadWaves == kSlotBlocks, "");

// Source offset of load i of this lane: LDS granule (i*4 + wave)*64 + lane of a
// slot is row tok = g / 72, physical granule g % 72, which holds logical granule
// (g % 72) ^ swz(tok).  Rows at or past `valid` repeat row valid-1, so bytes past
// a request's end are never read.
__device__ __forceinline__ int dma_off(int i, int wave, int lane, int valid) {
  const int gi = (i * kLoadWaves + wave) * 64 + lane;
  const int tok = gi / kGranPerRow;
  const int phys = gi - tok * kGranPerRow;
  const int src_tok = tok < valid ? tok : valid - 1;
  return src_tok * kRowBytes + ((phys ^ swz(tok)) << 4);
}

// All of this wave's direct-to-LDS loads of one chunk in one asm block: load i
// reads base + voff[i] into the 1 KiB LDS block m0 + 4096 i (block i*4 + wave).
// The wait states cover an SGPR base just written by VALU (5) and each M0
// update (1).
__device__ __forceinline__ void dma_chunk(const void* base, uint32_t m0, const int (&voff)[kLoadsPerWave]) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint64_t sbase = ((uint64_t)hi << 32) | (uint64_t)lo;
  uint32_t m = __builtin_amdgcn_readfirstlane(m0);
  asm volatile(
      "s_nop 4\n\t"
      "global_load_lds_dwordx4 %1, %10 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %10 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %10 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %4, %10 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %5, %10 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %6, %10 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %7, %10 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %8, %10 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %9, %10 nt"
      : "+{m0}"(m)
      : "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "v"(voff[4]), "v"(voff[5]), "v"(voff[6]),
        "v"(voff[7]), "v"(voff[8]), "s"(sbase)
      : "memory");
}


__global__ __launch_bounds__(kThreads, 1) void mla_decode_bf16_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kSlots * kSlotBytes];
  char LDS_AS* smem = (char LDS_AS*)(smem_raw);
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;   // row of this lane within the wave (and token row of the QK A-operand)
  const int q = lane >> 4;   // 16-lane group

  // blockIdx -> (stretch, row block).  Consecutive stretches (pieces of the same
  // request) are kept on one XCD: blocks are dealt to the 8 XCDs round robin,
  // so block i runs on XCD i % 8.
  const int nblk = gridDim.x;
  int lin = blockIdx.x;
  if ((nblk & 7) == 0) lin = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  const int stretch = lin / a.nrb;
  const int rb = lin - stretch * a.nrb;

  Header* hdr = reinterpret_cast<Header*>(a.ws + a.lay.header);
  const Header plan_hdr = load_const<Header>(a.ws + a.lay.header);
  const WgInfo wg = load_const<WgInfo>(a.ws + a.lay.wg_info + sizeof(WgInfo) * stretch);
  const char* reqs = a.ws + a.lay.req_info;
  if (!header_matches(plan_hdr, a.batch, a.rows, a.nwg, a.max_blocks)) {
    write_empty_rows(a, stretch, rb);
    return;
  }
  if (wg.page_begin >= wg.page_end) return;

  const int row_local = wave * kRowsPerWave + n;
  const int row = rb * kRowsPerBlock + row_local;
  const bool row_ok = row < a.rows;
  const int qi = row_ok ? row / a.num_heads : 0;   // which new token this row belongs to
  const bool loader = wave < kLoadWaves;

  // Per-lane LDS byte offsets within a slot.
  // QK A-operand: token 16tt + n, logical granule 4k + q -> physical 8(k>>1) + ((4(k&1)) ^ y).
  const int y = q ^ swz(n);
  const int qk_off0 = n * kRowBytes + ((0 ^ y) << 4);
  const int qk_off1 = n * kRowBytes + ((4 ^ y) << 4);
  // PV A-operand (V^T) through the transposing read: this lane supplies token
  // 4q + (lane>>2 & 3) (+16 for the second read) and dims 16d + 4(lane & 3),
  // i.e. logical granule 2d + (lane>>1 & 1) -> physical 8(d>>2) + ((2(d&3)) ^ z).
  int pv_off[4];
  {
    const int tr = 4 * q + ((lane >> 2) & 3);
    const int z = ((lane >> 1) & 1) ^ swz(tr);
#pragma unroll
    for (int dm = 0; dm < 4; dm++) pv_off[dm] = tr * kRowBytes + (((2 * dm) ^ z) << 4) + (lane & 1) * 8;
  }

  int gpage = wg.page_begin;
  int b = wg.b_begin;
  bool first_segment = true;
  while (gpage < wg.page_end && b < a.batch) {
    // Set-up of a segment is a chain of memory round trips, so the independent
    // loads go out together: the queries of request b, the block-table window
    // (its request-local first page comes from the plan, or is 0 for a later
    // segment) and the request's info.  Then chunks 0..2 are issued back to back.
    //
    // Queries: 18 B-fragments, q~[row][32k + 8q .. +8).
    bf16x8_t qf[kKSteps];
    {
      const bf16x8_t* qrow =
          reinterpret_cast<const bf16x8_t*>(a.q + ((size_t)b * a.rows + (row_ok ? row : 0)) * kHeadDimQK) + q;
#pragma unroll
      for (int k = 0; k < kKSteps; k++) {
        bf16x8_t v = qrow[4 * k];
        if (!row_ok) v = bf16x8_t{};
        qf[k] = v;
      }
    }
    const int pg0 = first_segment ? wg.pg0_local : 0;
    const int32_t* bt_row = a.block_table + (size_t)b * a.max_blocks;
    // Block-table window: lane i holds the page of request page pg0 + win + i,
    // so a chunk's page is one readlane rather than a scalar load waited on.
    // Entries past the request's pages (within its row) are loaded and unused.
    auto load_window = [&](int w) {
      const int pi = pg0 + w + opaque_lane();
      return pi < a.max_blocks ? bt_row[pi] : 0;
    };
    int win = 0;
    int win_pages = load_window(0);

    const ReqInfo rq = load_const<ReqInfo>(reqs + sizeof(ReqInfo) * b);
    if (rq.npages == 0) { b++; continue; }
    const int req_end = rq.page_first + rq.npages;
    const int pg1 = (wg.page_end < req_end ? wg.page_end : req_end) - rq.page_first;
    const int split = first_segment ? wg.ne_prefix - rq.ne_lo : 0;
    const int L = rq.seqlen;
    const int t_lo = pg0 * kPageSize;
    const int t_hi = pg1 * kPageSize < L ? pg1 * kPageSize : L;
    const int nchunks = (t_hi - t_lo + kChunk - 1) / kChunk;
    const int n_vis = a.causal ? L - a.seqlen_q + 1 + qi : L;      // keys this lane's row may see
    const int min_vis = a.causal ? L - a.seqlen_q + 1 : L;          // smallest over the request's rows
    const char* kv = reinterpret_cast<const char*>(a.kv);

    // The previous segment's readers of the slots are done.
    __syncthreads();

    auto issue = [&](int c) {
      if (!loader) return;
      const int t0 = t_lo + c * kChunk;
      int pw = (c >> 1) - win;   // t_lo is page aligned: two chunks per page
      if (pw >= 64) {
        win += 64;
        pw -= 64;
        win_pages = load_window(win);
        // Wait here, once per 64 pages: the compiler does not count the
        // inline-asm chunk loads, so it cannot tell that an older window load
        // has landed and would otherwise drain every load before each readlane.
        __builtin_amdgcn_s_waitcnt(VMCNT(0));
      }
      int page = __builtin_amdgcn_readlane(win_pages, pw);
      const bool bad = page < 0 || page >= a.num_pages;
      page = bad ? 0 : page;
      if (bad && tid == 0) atomicOr(&hdr->flags, 2u);
      const char* src = kv + ((size_t)page * kPageSize + (t0 % kPageSize)) * kRowBytes;
      const int valid = t_hi - t0 < kChunk ? t_hi - t0 : kChunk;
      const uint32_t m0 = smem_addr + (c % kSlots) * kSlotBytes + wave * 1024;
      // Per-lane offsets rebuilt from the lane at each issue (a few VALU on the
      // loading waves) rather than nine registers kept live.
      const int l = opaque_lane();
      int voff[kLoadsPerWave];
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; i++) voff[i] = dma_off(i, wave, l, valid);
      dma_chunk(src, m0, voff);
    };
    // Queries and window have landed before the first readlane.  Waiting here,
    // outside the issue loop, leaves the compiler nothing of its own to wait for
    // inside it, so the chunk loads stay in flight.
    __builtin_amdgcn_s_waitcnt(VMCNT(0));
    for (int c = 0; c < kSlots - 1 && c < nchunks; c++) issue(c);

    float m_ref = -INFINITY;   // reference maximum (log2 units), same in all lanes of a row
    float lsum = 0.f;          // this lane's part of the normaliser
    f32x4_t o[kDimTiles];
#pragma unroll
    for (int d = 0; d < kDimTiles; d++) o[d] = f32x4_t{};

    for (int c = 0; c < nchunks; c++) {
      // Wait until this wave's loads of chunk c have landed (later chunks may stay in flight).
      const int ahead = (nchunks - 1 < c + kSlots - 2 ? nchunks - 1 : c + kSlots - 2) - c;
      if (ahead >= 2) __builtin_amdgcn_s_waitcnt(VMCNT(18));
      else if (ahead == 1) __builtin_amdgcn_s_waitcnt(VMCNT(9));
      else __builtin_amdgcn_s_waitcnt(VMCNT(0));
      __syncthreads();   // every wave's part of chunk c is in LDS; slot (c-1)%4 is free
      if (c + kSlots - 1 < nchunks) issue(c + kSlots - 1);

      const char LDS_AS* slot = smem + (c % kSlots) * kSlotBytes;
      const int t0 = t_lo + c * kChunk;

      // S^T[token][row] over the 576 dims, two 16-token tiles.  Fragments are read
      // two K-steps ahead so each MFMA's operands are already in flight.
      f32x4_t s0 = f32x4_t{}, s1 = f32x4_t{};
      auto qk_off = [&](int kk) { return ((kk & 1) ? qk_off1 : qk_off0) + (kk >> 1) * 128; };
      bf16x8_t a0 = lds_read_b128(slot + qk_off(0));
      bf16x8_t a1 = lds_read_b128(slot + 16 * kRowBytes + qk_off(0));
      bf16x8_t b0 = lds_read_b128(slot + qk_off(1));
      bf16x8_t b1 = lds_read_b128(slot + 16 * kRowBytes + qk_off(1));
#pragma unroll
      for (int k = 0; k < kKSteps; k++) {
        bf16x8_t n0 = b0, n1 = b1;
        if (k + 2 < kKSteps) {
          n0 = lds_read_b128(slot + qk_off(k + 2));
          n1 = lds_read_b128(slot + 16 * kRowBytes + qk_off(k + 2));
        }
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[k], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[k], s1, 0, 0, 0);
        a0 = b0;
        a1 = b1;
        b0 = n0;
        b1 = n1;
        // keep steps k+1 and k+2's reads ahead of step k's MFMAs
        __builtin_amdgcn_sched_barrier(0);
      }

      // Mask, online softmax.  s0[i] is token 4q + i, s1[i] token 16 + 4q + i.
      // Keys at or past the row's visible length are set to -inf; only a
      // request's last chunk, or its causal tail, needs it (uniform branch).
      if (t0 + kChunk > min_vis) {
        const int lim = n_vis - t0 - 4 * q;   // token 4q + i visible if i < lim, 16 + 4q + i if 16 + i < lim
#pragma unroll
        for (int i = 0; i < 4; i++) {
          if (i >= lim) s0[i] = -INFINITY;
          if (16 + i >= lim) s1[i] = -INFINITY;
        }
      }
      // This lane's maximum over its 8 scores (the scale is positive, so it is
      // applied to the maximum).  Lazy rescale: nothing to do unless some score
      // exceeds the row's reference by more than 2^8; only then is the exact
      // row maximum formed and taken as the new reference.
      float cmax = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                         fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3]))) * a.scale_log2;
      if (__builtin_amdgcn_ballot_w64(cmax > m_ref + kLazyRescale)) {
        const float rmax = row_max(cmax);
        const float m_new = rmax > m_ref + kLazyRescale ? rmax : m_ref;
        const float alpha = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
        lsum *= alpha;
#pragma unroll
        for (int d = 0; d < kDimTiles; d++) o[d] *= alpha;
        m_ref = m_new;
      }
      const float mu = m_ref == -INFINITY ? 0.f : m_ref;
      bf16x8_t pb;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(i < 4 ? s0[i] : s1[i - 4], a.scale_log2, -mu));
        lsum += p;
        pb[i] = (__bf16)p;
      }

      // O^T[dim][row] += V^T[dim][token] . P^T[token][row], 32 tiles of 16 dims,
      // V^T fragments read three tiles ahead.
      auto read_v = [&](int d) {
        const int off = pv_off[d & 3] + (d >> 2) * 128;
        const i16x4_t lo = lds_read_tr16(slot + off);
        const i16x4_t hi = lds_read_tr16(slot + 16 * kRowBytes + off);
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8_t v0 = read_v(0), v1 = read_v(1), v2 = read_v(2);
#pragma unroll
      for (int d = 0; d < kDimTiles; d++) {
        bf16x8_t v3 = v2;
        if (d + 3 < kDimTiles) v3 = read_v(d + 3);
        o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v0, pb, o[d], 0, 0, 0);
        v0 = v1;
        v1 = v2;
        v2 = v3;
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // Finalise this segment: normalise, then write the output rows or a partial.
    // Addresses are rebuilt from the lane here rather than hoisted out of the
    // segment loop (64-bit pointers kept live across it would be spilled, and
    // every reload would wait for all outstanding stores).
    {
      const float ltot = row_sum(lsum);
      const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
      const float lse_v = ltot > 0.f ? (m_ref + __builtin_amdgcn_logf(ltot)) * kLn2 : -INFINITY;
      const int ol = opaque_lane();
      const int orow_local = wave * kRowsPerWave + (ol & 15);
      const int orow_g = rb * kRowsPerBlock + orow_local;
      const int oq = ol >> 4;
      if (rq.nsplit <= 1) {
        if (orow_g < a.rows) {
          uint16_t* orow = a.out + ((size_t)b * a.rows + orow_g) * kHeadDimV + 4 * oq;
#pragma unroll
          for (int d = 0; d < kDimTiles; d++) {
            bf16x4_t w;
#pragma unroll
            for (int r = 0; r < 4; r++) w[r] = (__bf16)(o[d][r] * inv);
            *reinterpret_cast<bf16x4_t*>(orow + 16 * d) = w;
          }
          if (oq == 0) a.lse[(size_t)b * a.rows + orow_g] = lse_v;
        }
      } else {
        const int slot_id = rq.slot_off + split;
        if (slot_id >= 0 && slot_id < 2 * a.nwg)   // uniform
          store_partial(a, ((size_t)slot_id * a.nrb + rb) * kRowsPerBlock, smem, o, inv, lse_v);
      }
    }
    gpage = rq.page_first + pg1;
    b++;
    first_segment = false;
  }
}

// ---------------------------------------------------------------------------
// FP8 (E4M3FN) cache with one fp32 scale per token: kv_t = decode(code_t) * scale_t.
// The codes are widened to bf16 exactly (every E4M3FN value is a bf16 value)
// and fed to the same bf16 MFMAs; the scale is applied where it is exact in
// fp32 -- to column t of the scores, and to p_t before P is rounded to bf16 for
// the P . V product.  The normaliser sums the unscaled p_t.
//
// A chunk of 32 tokens arrives as codes in a 4-slot ring (half the bytes of a
// bf16 chunk, so four chunks are in flight in 74 KiB).  Once it has landed the
// whole workgroup widens it, in one pass, into one of two bf16 buffers laid out
// as a bf16 slot; the score and value loops of the bf16 kernel then read it
// unchanged.  Widening once per chunk costs 1,152 conversions per workgroup,
// where widening at each read would repeat them in every wave's fragments.
// ---------------------------------------------------------------------------
constexpr int kRowBytes8 = kHeadDimQK;                  // 576 one-byte codes per token
constexpr int kChunk8 = 32;                             // tokens per slot
constexpr int kSlots8 = 4;                              // ring depth (chunks c+1 .. c+4 around iteration c)
constexpr int kSlotBytes8 = kChunk8 * kRowBytes8;       // 18432
constexpr int kSlotBlocks8 = kSlotBytes8 / 1024;        // 18 one-KiB loads
constexpr int kGranPerRow8 = kRowBytes8 / 16;           // 36
constexpr int kScaleBytes8 = kChunk8 * 4;               // 128 bytes of scales per slot
constexpr int kRingBytes8 = kSlots8 * (kSlotBytes8 + kScaleBytes8);   // 74,240
// Widened chunks: two bf16 buffers in the bf16 kernel's slot layout, 1 KiB aligned,
// then the two chunks' token scales.
constexpr int kWideOff8 = (kRingBytes8 + 1023) / 1024 * 1024;
constexpr int kWideScaleOff8 = kWideOff8 + 2 * kSlotBytes;
constexpr int kLdsBytes8 = kWideScaleOff8 + 2 * kScaleBytes8;
static_assert(kLdsBytes8 <= 160 * 1024, "FP8 ring must fit in 160 KiB");
static_assert(kSlotBlocks8 + 1 <= 3 * kWaves, "slot loads (codes + one scale block) fit three per wave");

// Loads per wave per slot: 18 code blocks and one scale block over 8 waves.
__device__ __forceinline__ int dma_per_slot8(int wave) { return wave < 3 ? 3 : 2; }

// Part i of a slot fill: block i*8 + wave.  Blocks 0..17 carry 32 token rows of
// codes in cache order (granule g of the slot is token g / 36, granule g % 36);
// block 18 carries the 32 scales (8 lanes x 4).  Rows at or past `valid` repeat
// row valid-1.
__device__ __forceinline__ void load_chunk_part8(const char* src, const float* scale_src, int valid,
                                                 uint32_t slot_lds, uint32_t scale_lds, int i, int wave, int lane) {
  const int blk = i * kWaves + wave;
  if (blk < kSlotBlocks8) {
    const int gi = blk * 64 + lane;
    const int tok = gi / kGranPerRow8;
    const int phys = gi - tok * kGranPerRow8;
    const int src_tok = tok < valid ? tok : valid - 1;
    dma16(src, (uint32_t)(src_tok * kRowBytes8 + (phys << 4)), slot_lds + blk * 1024);
  } else if (blk == kSlotBlocks8 && lane < kChunk8 / 4) {
    dma16(scale_src, (uint32_t)(lane * 16), scale_lds);
  }
}

// Four E4M3FN codes (one dword) -> four bf16, exactly.
__device__ __forceinline__ void fp8x4_to_bf16(uint32_t w, bf16x8_t& out, int at) {
  const auto lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const auto hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  out[at + 0] = lo[0];
  out[at + 1] = lo[1];
  out[at + 2] = hi[0];
  out[at + 3] = hi[1];
}

typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads, 1) void mla_decode_fp8_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kLdsBytes8];
  char LDS_AS* smem = (char LDS_AS*)(smem_raw);
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;
  const uint32_t scale_addr = smem_addr + kSlots8 * kSlotBytes8;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int q = lane >> 4;

  const int nblk = gridDim.x;
  int lin = blockIdx.x;
  if ((nblk & 7) == 0) lin = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  const int stretch = lin / a.nrb;
  const int rb = lin - stretch * a.nrb;

  Header* hdr = reinterpret_cast<Header*>(a.ws + a.lay.header);
  const Header plan_hdr = load_const<Header>(a.ws + a.lay.header);
  const WgInfo wg = load_const<WgInfo>(a.ws + a.lay.wg_info + sizeof(WgInfo) * stretch);
  const char* reqs = a.ws + a.lay.req_info;
  if (!header_matches(plan_hdr, a.batch, a.rows, a.nwg, a.max_blocks)) {
    write_empty_rows(a, stretch, rb);
    return;
  }
  if (wg.page_begin >= wg.page_end) return;

  const int row_local = wave * kRowsPerWave + n;
  const int row = rb * kRowsPerBlock + row_local;
  const bool row_ok = row < a.rows;
  const int qi = row_ok ? row / a.num_heads : 0;
  const int ndma = dma_per_slot8(wave);

  // Reads of a widened chunk: the bf16 kernel's slot layout and offsets.
  const int y = q ^ swz(n);
  const int qk_off0 = n * kRowBytes + ((0 ^ y) << 4);
  const int qk_off1 = n * kRowBytes + ((4 ^ y) << 4);
  int pv_off[4];
  {
    const int tr = 4 * q + ((lane >> 2) & 3);
    const int z = ((lane >> 1) & 1) ^ swz(tr);
#pragma unroll
    for (int dm = 0; dm < 4; dm++) pv_off[dm] = tr * kRowBytes + (((2 * dm) ^ z) << 4) + (lane & 1) * 8;
  }

  // Widening of one chunk by the whole workgroup: 1,152 granules of 16 codes, up
  // to three per thread (64 consecutive granules per wave read: conflict free).
  // FP8 granule g of the slot is token g / 36, granule j = g % 36 (dims 16 j ..
  // +15); its two halves become bf16 logical granules 2 j and 2 j + 1 of the
  // token's 1,152-byte row, stored at physical granule (logical ^ swz(token)).
  // The chunk's 32 token scales are copied beside it.
  auto widen = [&](int cw) {
    const char LDS_AS* src = smem + (cw % kSlots8) * kSlotBytes8;
    char LDS_AS* dst = smem + kWideOff8 + (cw & 1) * kSlotBytes;
    // The thread index, hidden from the optimiser: the addresses below are
    // recomputed per chunk (a few VALU) instead of kept live across the loop.
    int tid_o = (int)threadIdx.x;
    asm volatile("" : "+v"(tid_o));
#pragma unroll
    for (int u = 0; u < 3; u++) {
      const int g = tid_o + kThreads * u;
      if (g < kSlotBytes8 / 16) {
        const int tok = g / kGranPerRow8;
        const int j = g - tok * kGranPerRow8;
        const i32x4_t w = *reinterpret_cast<const i32x4_t LDS_AS*>(src + 16 * g);
        bf16x8_t lo, hi;
        fp8x4_to_bf16((uint32_t)w[0], lo, 0);
        fp8x4_to_bf16((uint32_t)w[1], lo, 4);
        fp8x4_to_bf16((uint32_t)w[2], hi, 0);
        fp8x4_to_bf16((uint32_t)w[3], hi, 4);
        const int sw = swz(tok);
        *reinterpret_cast<bf16x8_t LDS_AS*>(dst + tok * kRowBytes + (((2 * j) ^ sw) << 4)) = lo;
        *reinterpret_cast<bf16x8_t LDS_AS*>(dst + tok * kRowBytes + (((2 * j + 1) ^ sw) << 4)) = hi;
      }
    }
    if (tid_o < kScaleBytes8 / 16) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t LDS_AS*>(smem + kSlots8 * kSlotBytes8 +
                                                                 (cw % kSlots8) * kScaleBytes8 + 16 * tid_o);
      *reinterpret_cast<f32x4_t LDS_AS*>(smem + kWideScaleOff8 + (cw & 1) * kScaleBytes8 + 16 * tid_o) = v;
    }
  };

  int gpage = wg.page_begin;
  int b = wg.b_begin;
  bool first_segment = true;
  while (gpage < wg.page_end && b < a.batch) {
    // Set-up as in the bf16 kernel: queries, block-table window and request
    // info go out together, then chunks 0..3.
    // Queries (natural order: the widened chunk has the bf16 layout).
    bf16x8_t qf[kKSteps];
    {
      const bf16x8_t* qrow =
          reinterpret_cast<const bf16x8_t*>(a.q + ((size_t)b * a.rows + (row_ok ? row : 0)) * kHeadDimQK) + q;
#pragma unroll
      for (int k = 0; k < kKSteps; k++) {
        bf16x8_t v = qrow[4 * k];
        if (!row_ok) v = bf16x8_t{};
        qf[k] = v;
      }
    }
    const int pg0 = first_segment ? wg.pg0_local : 0;
    const int32_t* bt_row = a.block_table + (size_t)b * a.max_blocks;
    auto load_window = [&](int w) {
      const int pi = pg0 + w + opaque_lane();
      return pi < a.max_blocks ? bt_row[pi] : 0;
    };
    int win = 0;
    int win_pages = load_window(0);

    const ReqInfo rq = load_const<ReqInfo>(reqs + sizeof(ReqInfo) * b);
    if (rq.npages == 0) { b++; continue; }
    const int req_end = rq.page_first + rq.npages;
    const int pg1 = (wg.page_end < req_end ? wg.page_end : req_end) - rq.page_first;
    const int split = first_segment ? wg.ne_prefix - rq.ne_lo : 0;
    const int L = rq.seqlen;
    const int t_lo = pg0 * kPageSize;
    const int t_hi = pg1 * kPageSize < L ? pg1 * kPageSize : L;
    const int nchunks = (t_hi - t_lo + kChunk8 - 1) / kChunk8;
    const int n_vis = a.causal ? L - a.seqlen_q + 1 + qi : L;
    const int min_vis = a.causal ? L - a.seqlen_q + 1 : L;
    const char* kv = reinterpret_cast<const char*>(a.kv);

    // The previous segment's readers of the slots and buffers are done.
    __syncthreads();

    auto issue = [&](int c) {
      const int t0 = t_lo + c * kChunk8;
      int pw = (c >> 1) - win;   // t_lo is page aligned: two chunks per page
      if (pw >= 64) {
        win += 64;
        pw -= 64;
        win_pages = load_window(win);
        __builtin_amdgcn_s_waitcnt(VMCNT(0));   // as in the bf16 kernel
      }
      int page = __builtin_amdgcn_readlane(win_pages, pw);
      const bool bad = page < 0 || page >= a.num_pages;
      page = bad ? 0 : page;
      if (bad && tid == 0) atomicOr(&hdr->flags, 2u);
      const size_t tok0 = (size_t)page * kPageSize + (t0 % kPageSize);
      const char* src = kv + tok0 * kRowBytes8;
      const float* ssrc = a.kv_scale + tok0;
      const int valid = t_hi - t0 < kChunk8 ? t_hi - t0 : kChunk8;
      const int slot = c % kSlots8;
#pragma unroll
      for (int i = 0; i < 3; i++)
        if (i < ndma)
          load_chunk_part8(src, ssrc, valid, smem_addr + slot * kSlotBytes8, scale_addr + slot * kScaleBytes8, i,
                           wave, lane);
    };
    __builtin_amdgcn_s_waitcnt(VMCNT(0));   // queries and window (as in the bf16 kernel)
    for (int c = 0; c < kSlots8 && c < nchunks; c++) issue(c);
    {
      // Wait for this wave's loads of chunk 0; chunks 1..3 may stay in flight.
      const int after0 = nchunks - 1 < kSlots8 - 1 ? nchunks - 1 : kSlots8 - 1;
      if (ndma == 3) {
        if (after0 >= 3) __builtin_amdgcn_s_waitcnt(VMCNT(9));
        else if (after0 == 2) __builtin_amdgcn_s_waitcnt(VMCNT(6));
        else if (after0 == 1) __builtin_amdgcn_s_waitcnt(VMCNT(3));
        else __builtin_amdgcn_s_waitcnt(VMCNT(0));
      } else {
        if (after0 >= 3) __builtin_amdgcn_s_waitcnt(VMCNT(6));
        else if (after0 == 2) __builtin_amdgcn_s_waitcnt(VMCNT(4));
        else if (after0 == 1) __builtin_amdgcn_s_waitcnt(VMCNT(2));
        else __builtin_amdgcn_s_waitcnt(VMCNT(0));
      }
    }
    __syncthreads();   // chunk 0's codes are in LDS
    widen(0);

    float m_ref = -INFINITY;
    float lsum = 0.f;
    f32x4_t o[kDimTiles];
#pragma unroll
    for (int d = 0; d < kDimTiles; d++) o[d] = f32x4_t{};

    for (int c = 0; c < nchunks; c++) {
      // Wait for this wave's loads of chunk c+1; chunks up to c+3 may stay in flight.
      const int ahead = c + 1 < nchunks ? (nchunks - 1 < c + 3 ? nchunks - 1 : c + 3) - (c + 1) : 0;
      if (ndma == 3) {
        if (ahead >= 2) __builtin_amdgcn_s_waitcnt(VMCNT(6));
        else if (ahead == 1) __builtin_amdgcn_s_waitcnt(VMCNT(3));
        else __builtin_amdgcn_s_waitcnt(VMCNT(0));
      } else {
        if (ahead >= 2) __builtin_amdgcn_s_waitcnt(VMCNT(4));
        else if (ahead == 1) __builtin_amdgcn_s_waitcnt(VMCNT(2));
        else __builtin_amdgcn_s_waitcnt(VMCNT(0));
      }
      // Chunk c is widened; chunk c+1's codes are in LDS; slot c % 4 and widened
      // buffer (c+1) & 1 were last read before this barrier.
      __syncthreads();
      if (c + kSlots8 < nchunks) issue(c + kSlots8);
      if (c + 1 < nchunks) widen(c + 1);

      const char LDS_AS* slot = smem + kWideOff8 + (c & 1) * kSlotBytes;
      const float LDS_AS* sc_lds = (const float LDS_AS*)(smem + kWideScaleOff8 + (c & 1) * kScaleBytes8);
      const int t0 = t_lo + c * kChunk8;

      // S^T[token][row] over the 576 dims (the bf16 kernel's loop on the widened chunk).
      f32x4_t s0 = f32x4_t{}, s1 = f32x4_t{};
      bf16x8_t a0 = lds_read_b128(slot + qk_off0);
      bf16x8_t a1 = lds_read_b128(slot + 16 * kRowBytes + qk_off0);
#pragma unroll
      for (int k = 0; k < kKSteps; k++) {
        bf16x8_t n0 = a0, n1 = a1;
        if (k + 1 < kKSteps) {
          const int off = (((k + 1) & 1) ? qk_off1 : qk_off0) + ((k + 1) >> 1) * 128;
          n0 = lds_read_b128(slot + off);
          n1 = lds_read_b128(slot + 16 * kRowBytes + off);
        }
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[k], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[k], s1, 0, 0, 0);
        a0 = n0;
        a1 = n1;
        __builtin_amdgcn_sched_barrier(0);
      }

      // Token scales of this lane's eight tokens: 4q + i and 16 + 4q + i.
      const f32x4_t sc0 = *reinterpret_cast<const f32x4_t LDS_AS*>(sc_lds + 4 * q);
      const f32x4_t sc1 = *reinterpret_cast<const f32x4_t LDS_AS*>(sc_lds + 16 + 4 * q);
      float x[8], w[8];   // scaled scores (before the softmax scale) and p's token scale
#pragma unroll
      for (int i = 0; i < 8; i++) {
        w[i] = i < 4 ? sc0[i] : sc1[i - 4];
        x[i] = (i < 4 ? s0[i] : s1[i - 4]) * w[i];
      }
      // Keys at or past the row's visible length get score -inf and weight scale 0
      // (a scale past a request's end may be anything, NaN included).
      if (t0 + kChunk8 > min_vis) {
        const int lim = n_vis - t0 - 4 * q;
#pragma unroll
        for (int i = 0; i < 8; i++)
          if (16 * (i >> 2) + (i & 3) >= lim) {
            x[i] = -INFINITY;
            w[i] = 0.f;
          }
      }
      float cmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7]))) *
                   a.scale_log2;
      if (__builtin_amdgcn_ballot_w64(cmax > m_ref + kLazyRescale)) {
        const float rmax = row_max(cmax);
        const float m_new = rmax > m_ref + kLazyRescale ? rmax : m_ref;
        const float alpha = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
        lsum *= alpha;
#pragma unroll
        for (int d = 0; d < kDimTiles; d++) o[d] *= alpha;
        m_ref = m_new;
      }
      const float mu = m_ref == -INFINITY ? 0.f : m_ref;
      bf16x8_t pb;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], a.scale_log2, -mu));
        lsum += p;
        pb[i] = (__bf16)(p * w[i]);
      }

      // O^T += V^T . P'^T (the bf16 kernel's loop on the widened chunk).
      auto read_v = [&](int d) {
        const int off = pv_off[d & 3] + (d >> 2) * 128;
        const i16x4_t lo = lds_read_tr16(slot + off);
        const i16x4_t hi = lds_read_tr16(slot + 16 * kRowBytes + off);
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8_t v0 = read_v(0), v1 = read_v(1);
#pragma unroll
      for (int d = 0; d < kDimTiles; d++) {
        bf16x8_t v2 = v1;
        if (d + 2 < kDimTiles) v2 = read_v(d + 2);
        o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v0, pb, o[d], 0, 0, 0);
        v0 = v1;
        v1 = v2;
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // Finalise: addresses rebuilt from the lane (see the bf16 kernel).
    {
      const float ltot = row_sum(lsum);
      const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
      const float lse_v = ltot > 0.f ? (m_ref + __builtin_amdgcn_logf(ltot)) * kLn2 : -INFINITY;
      const int ol = opaque_lane();
      const int orow_local = wave * kRowsPerWave + (ol & 15);
      const int orow_g = rb * kRowsPerBlock + orow_local;
      const int oq = ol >> 4;
      if (rq.nsplit <= 1) {
        if (orow_g < a.rows) {
          uint16_t* orow = a.out + ((size_t)b * a.rows + orow_g) * kHeadDimV + 4 * oq;
#pragma unroll
          for (int d = 0; d < kDimTiles; d++) {
            bf16x4_t wv;
#pragma unroll
            for (int r = 0; r < 4; r++) wv[r] = (__bf16)(o[d][r] * inv);
            *reinterpret_cast<bf16x4_t*>(orow + 16 * d) = wv;
          }
          if (oq == 0) a.lse[(size_t)b * a.rows + orow_g] = lse_v;
        }
      } else {
        const int slot_id = rq.slot_off + split;
        if (slot_id >= 0 && slot_id < 2 * a.nwg)   // uniform
          store_partial(a, ((size_t)slot_id * a.nrb + rb) * kRowsPerBlock, smem, o, inv, lse_v);
      }
    }
    gpage = rq.page_first + pg1;
    b++;
    first_segment = false;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, bool fp8, hipStream_t stream) {
  void* args[] = {(void*)&a};
  const void* kern = fp8 ? (const void*)mla_decode_fp8_kernel : (const void*)mla_decode_bf16_kernel;
  return hipLaunchKernel(kern, dim3(a.nwg * a.nrb), dim3(kThreads), args, 0, stream);
}

}  // namespace mla
