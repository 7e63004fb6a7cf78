// mla_workspace.h -- layout of the caller-owned workspace shared by the plan,
// decode and combine kernels of libmla_decode.  Internal to the library.
#pragma once

#include <stddef.h>
#include <stdint.h>

#ifndef MLA_HD
#define MLA_HD
#endif

namespace mla {

constexpr int kHeadDimQK = 576;     // 512 latent + 64 RoPE numbers per cached token
constexpr int kHeadDimV = 512;      // the latent part is the value
constexpr int kPageSize = 64;       // tokens per page
constexpr int kRowsPerBlock = 128;  // query rows one workgroup holds (8 waves x 16)
constexpr int kMaxHeads = 128;
constexpr int kMaxSeqlenQ = 8;
constexpr int kMaxBatch = 8192;      // requests per step (the plan keeps its arrays in LDS)
constexpr int kMaxStretches = 4096;  // persistent workgroups per row block
constexpr int kPlanCostPerRequest = 3;  // fixed cost of a request segment (set-up + finalise), in pages
constexpr uint32_t kMagic = 0x4D4C4131u;  // "MLA1"

MLA_HD inline int row_blocks(int rows) { return (rows + kRowsPerBlock - 1) / kRowsPerBlock; }

// Per persistent workgroup (stretch) of the plan.
struct WgInfo {
  int32_t page_begin;  // first page (global position in the concatenation of all requests' pages)
  int32_t page_end;    // one past the last page
  int32_t b_begin;     // request that holds page_begin
  int32_t ne_prefix;   // number of non-empty stretches before this one
  int32_t pg0_local;   // page_begin - page_first of b_begin: lets the decode load the block-table
                       // window before the request's info arrives (0 for an empty stretch)
  int32_t pad[3];
};

// Per request.
struct ReqInfo {
  int32_t page_first;  // global position of the request's first page
  int32_t npages;      // pages the request uses (ceil(L / 64) of the clamped L)
  int32_t nsplit;      // stretches that hold part of the request (1: written directly)
  int32_t slot_off;    // first partial slot of the request (nsplit > 1)
  int32_t ne_lo;       // ne_prefix of the first stretch that holds the request
  int32_t seqlen;      // L after clamping to [0, max_blocks * 64]
  int32_t pad0, pad1;
};

struct Header {
  uint32_t magic;
  uint32_t flags;       // MLA_FLAG_* bits
  int32_t batch;
  int32_t rows;         // seqlen_q * num_heads
  int32_t nwg;          // stretches
  int32_t nrb;          // row blocks of 128 per request
  int32_t max_slots;    // partial slots reserved (2 * nwg)
  int32_t total_pages;
  int32_t used_slots;
  int32_t max_blocks;   // row stride of the block table the plan clamped lengths to
  int32_t seqlen_q;
  int32_t pad[5];
};

// The decode and combine kernels trust the plan only when the header matches
// their own parameters (one scalar load of the header per workgroup).
MLA_HD inline bool header_matches(const Header& h, int batch, int rows, int nwg, int max_blocks) {
  return h.magic == kMagic && h.batch == batch && h.rows == rows && h.nwg == nwg && h.nrb == row_blocks(rows) &&
         h.max_slots == 2 * nwg && h.max_blocks == max_blocks;
}

// Byte offsets of every region; all 256-byte aligned.  A split request's piece
// is stored per row as an LSE, a power-of-two scale s and the normalised output
// divided by s in fp16 (|O / s| < 2^15: no overflow; the scaling is exact).
struct Layout {
  size_t header, wg_info, req_info, part_lse, part_scale, part_out, total;
};

MLA_HD inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }


MLA_HD inline Layout make_layout(int batch, int rows, int nwg) {
  Layout l;
  const int nrb = row_blocks(rows);
  const size_t slots = size_t(2) * nwg;
  size_t off = 0;
  l.header = off;   off = align256(off + sizeof(Header));
  l.wg_info = off;  off = align256(off + sizeof(WgInfo) * size_t(nwg));
  l.req_info = off; off = align256(off + sizeof(ReqInfo) * size_t(batch));
  l.part_lse = off;   off = align256(off + sizeof(float) * slots * nrb * kRowsPerBlock);
  l.part_scale = off; off = align256(off + sizeof(float) * slots * nrb * kRowsPerBlock);
  l.part_out = off;   off = align256(off + sizeof(uint16_t) * slots * nrb * kRowsPerBlock * kHeadDimV);
  l.total = off;
  return l;
}

}  // namespace mla
