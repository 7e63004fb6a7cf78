// mla_plan.hip -- split plan for MLA decode: which stretch of the paged KV each
// persistent workgroup handles.
//
// The pages of all requests are laid end to end.  Each request costs its page
// count plus a fixed per-request cost (loading its queries and writing its
// output), and the concatenation is cut into nwg stretches of equal cost.  A
// stretch boundary that falls inside a request splits it; the pieces are merged
// by their LSE afterwards.  This follows the scheduling metadata of the FlashMLA
// paragraph of "MLA inference: two computation paths and FlashMLA" (computed once
// from the context lengths, deciding which stretch of KV each compute unit
// handles) and the FlashMLA guide's "Native Ragged Sequence Batching" (work
// assigned by context length so long and short requests share the GPU).
//
// One workgroup of 256 threads does the whole plan on the device from the
// device-resident sequence lengths, so no host synchronisation is needed.  All
// working arrays live in LDS (batch <= kMaxBatch, stretches <= kMaxStretches),
// so every binary search is a handful of LDS reads.  The plan sits on the
// critical path of every step, so it is written for latency: the lengths are
// read from global memory once, and each phase costs one or two barriers.
#include <hip/hip_runtime.h>

#define MLA_HD __host__ __device__
#include "mla_launch.h"
#include "mla_workspace.h"

namespace mla {
namespace {

constexpr int kPlanThreads = 256;
constexpr int kPlanWaves = kPlanThreads / 64;

// Inclusive scan of four values over the workgroup with one pair of barriers;
// `wsum` is scratch for the per-wave totals.  Returns this thread's inclusive
// prefixes; *total receives the workgroup totals.
__device__ int4 block_scan4(int4 v, int4* wsum, int4* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int yx = __shfl_up(v.x, off, 64), yy = __shfl_up(v.y, off, 64);
    const int yz = __shfl_up(v.z, off, 64), yw = __shfl_up(v.w, off, 64);
    if (lane >= off) {
      v.x += yx;
      v.y += yy;
      v.z += yz;
      v.w += yw;
    }
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  int4 pre = make_int4(0, 0, 0, 0), tot = make_int4(0, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < kPlanWaves; i++) {   // a handful of waves: read the totals directly
    const int4 x = wsum[i];
    if (i < w) {
      pre.x += x.x;
      pre.y += x.y;
      pre.z += x.z;
      pre.w += x.w;
    }
    tot.x += x.x;
    tot.y += x.y;
    tot.z += x.z;
    tot.w += x.w;
  }
  *total = tot;
  __syncthreads();
  return make_int4(v.x + pre.x, v.y + pre.y, v.z + pre.z, v.w + pre.w);
}

// Largest power of two <= n (n >= 1).
__device__ int pow2_floor(int n) { return 1 << (31 - __builtin_clz(n)); }

// Largest index i in [0, n) with key(i) <= x, or -1 (key nondecreasing), by
// binary lifting: one dependent LDS read per halving of the step.
template <typename F>
__device__ int last_le(int n, int x, F key) {
  int pos = -1;
  for (int step = n > 0 ? pow2_floor(n) : 0; step > 0; step >>= 1)
    if (pos + step < n && key(pos + step) <= x) pos += step;
  return pos;
}

// floor(a * b / d) for 0 <= a, b, 0 < d, a * b < 2^53: the double quotient is
// within one of the exact one, and one integer step on each side corrects it.
__device__ int floor_muldiv(int a, int b, int d) {
  const int64_t num = (int64_t)a * b;
  int64_t q = (int64_t)((double)num / (double)d);
  if (q * d > num) q--;
  else if ((q + 1) * d <= num) q++;
  return (int)q;
}

__global__ __launch_bounds__(kPlanThreads) void mla_plan_kernel(const int32_t* __restrict__ seqlens, char* ws,
                                                                Layout lay, int batch, int seqlen_q, int rows,
                                                                int nwg, int max_blocks) {
  __shared__ int s_cost[kMaxBatch];        // exclusive prefix of per-request cost
  __shared__ int s_first[kMaxBatch];       // first page (global position) of each request
  __shared__ int s_len[kMaxBatch];         // clamped length of each request
  __shared__ int s_bnd[kMaxStretches + 1];   // stretch boundaries in page positions
  __shared__ int s_bb[kMaxStretches];        // request that holds each stretch's first page
  __shared__ int s_ne[kMaxStretches + 1];    // non-empty stretches before each stretch
  __shared__ int4 wsum[kPlanWaves];

  Header* hdr = reinterpret_cast<Header*>(ws + lay.header);
  WgInfo* wgi = reinterpret_cast<WgInfo*>(ws + lay.wg_info);
  ReqInfo* req = reinterpret_cast<ReqInfo*>(ws + lay.req_info);
  const int t = threadIdx.x;
  const int max_len = max_blocks * kPageSize;
  auto npages_of = [](int L) { return (L + kPageSize - 1) / kPageSize; };

  auto clamp_len = [&](int L) { return L < 0 ? 0 : (L > max_len ? max_len : L); };
  const int np0 = npages_of(clamp_len(seqlens[0]));

  // 1. pages and cost per request; exclusive prefix sums of both, a count of
  //    lengths outside [seqlen_q, max_len], and a count of requests whose page
  //    count differs from request 0's (none: every request has the same length).
  int carry_p = 0, carry_c = 0, nbad = 0, ndiff = 0;
  for (int base = 0; base < batch; base += kPlanThreads) {
    const int b = base + t;
    int L = 0, bad = 0;
    if (b < batch) {
      L = seqlens[b];
      bad = (L < seqlen_q || L > max_len) ? 1 : 0;
      L = clamp_len(L);
    }
    const int np = npages_of(L);
    const int cost = np > 0 ? np + kPlanCostPerRequest : 0;
    const int diff = (b < batch && np != np0) ? 1 : 0;
    int4 tot;
    const int4 inc = block_scan4(make_int4(np, cost, bad, diff), wsum, &tot);
    if (b < batch) {
      s_first[b] = carry_p + inc.x - np;
      s_cost[b] = carry_c + inc.y - cost;
      s_len[b] = L;
    }
    carry_p += tot.x;
    carry_c += tot.y;
    nbad += tot.z;
    ndiff += tot.w;
  }
  const int total_pages = carry_p;
  const int total_cost = carry_c;
  __syncthreads();

  // 2. stretch boundaries in page positions: boundary s sits at cost s * T / nwg,
  //    inside the last request b whose cost range starts at or before it.
  //    Lengths that differ: b's fixed cost sits before its pages, and a boundary
  //    inside it moves to b's first page (a stretch that takes a short request
  //    whole pays its set-up once, and no sliver of it is split off).  Equal
  //    lengths: every request is split the same way and every piece pays its
  //    own set-up, so b's fixed cost is spread evenly over its pages and the cut
  //    goes to the page nearest to (s T / nwg - cost_b) * np_b / (np_b + c); with
  //    the fixed cost in front, the first piece of each request came out c pages
  //    short (64 pages over four stretches: 13/17/17/17 rather than 16 each).
  const bool uniform = ndiff == 0;
  for (int s = t; s <= nwg; s += kPlanThreads) {
    if (s == nwg) {
      s_bnd[s] = total_pages;
    } else {
      const int x = floor_muldiv(s, total_cost, nwg);
      const int b = last_le(batch, x, [&](int i) { return s_cost[i]; });
      const int np = npages_of(s_len[b]);
      int k;
      if (uniform) {
        const double y = (double)s * (double)total_cost / (double)nwg - (double)s_cost[b];
        k = (int)floor(y * np / (double)(np + kPlanCostPerRequest) + 0.5);
      } else {
        k = x - s_cost[b] - kPlanCostPerRequest;
      }
      k = k < 0 ? 0 : (k > np ? np : k);
      const int bnd = s_first[b] + k;
      s_bnd[s] = bnd;
      // The request holding page bnd: b, unless the cut fell at b's end; none
      // when bnd is past the last page (then the stretch is empty).
      s_bb[s] = bnd >= total_pages ? batch
                : (k < np ? b : last_le(batch, bnd, [&](int i) { return s_first[i]; }));
    }
  }
  __syncthreads();

  // 3. non-empty stretches: exclusive prefix count, written with each stretch's info.
  {
    int carry = 0;
    for (int base = 0; base < nwg; base += kPlanThreads) {
      const int s = base + t;
      const int pb = s < nwg ? s_bnd[s] : 0;
      const int pe = s < nwg ? s_bnd[s + 1] : 0;
      const int ne = pe > pb ? 1 : 0;
      int4 tot;
      const int inc = block_scan4(make_int4(ne, 0, 0, 0), wsum, &tot).x;
      if (s < nwg) {
        const int ex = carry + inc - ne;
        s_ne[s] = ex;
        WgInfo w;
        const int bb = s_bb[s];
        w.page_begin = pb;
        w.page_end = pe;
        w.b_begin = bb;
        w.ne_prefix = ex;
        w.pg0_local = bb < batch ? pb - s_first[bb] : 0;
        w.pad[0] = w.pad[1] = w.pad[2] = 0;
        wgi[s] = w;
      }
      carry += tot.x;
    }
    if (t == 0) s_ne[nwg] = carry;
  }
  __syncthreads();

  // 4. per request: how many stretches hold it, and its partial slots.  The two
  //    searches (first stretch ending past the request's first page, last stretch
  //    beginning before its end) run interleaved.
  const int top = pow2_floor(nwg);
  int carry = 0;
  for (int base = 0; base < batch; base += kPlanThreads) {
    const int b = base + t;
    int nsplit = 0, ne_lo = 0, first = 0, L = 0;
    if (b < batch) {
      first = s_first[b];
      L = s_len[b];
      const int np = npages_of(L);
      if (np > 0) {
        const int last = first + np - 1;
        int lo = -1, hi = -1;
        for (int step = top; step > 0; step >>= 1) {
          const int i1 = lo + step, i2 = hi + step;
          if (i1 < nwg && s_bnd[i1 + 1] <= first) lo = i1;
          if (i2 < nwg && s_bnd[i2] <= last) hi = i2;
        }
        const int s_lo = lo + 1, s_hi = hi;
        nsplit = s_ne[s_hi + 1] - s_ne[s_lo];
        ne_lo = s_ne[s_lo];
      }
    }
    const int slots = nsplit > 1 ? nsplit : 0;
    int4 tot;
    const int inc = block_scan4(make_int4(slots, 0, 0, 0), wsum, &tot).x;
    if (b < batch) {
      ReqInfo r;
      r.page_first = first;
      r.npages = npages_of(L);
      r.nsplit = nsplit;
      r.slot_off = carry + inc - slots;
      r.ne_lo = ne_lo;
      r.seqlen = L;
      r.pad0 = r.pad1 = 0;
      req[b] = r;
    }
    carry += tot.x;
  }
  if (t == 0) {
    Header h;
    h.magic = kMagic;
    h.flags = nbad > 0 ? 1u : 0u;
    h.batch = batch;
    h.rows = rows;
    h.nwg = nwg;
    h.nrb = row_blocks(rows);
    h.max_slots = 2 * nwg;
    h.total_pages = total_pages;
    h.used_slots = carry;
    h.max_blocks = max_blocks;
    h.seqlen_q = seqlen_q;
    for (int i = 0; i < 5; i++) h.pad[i] = 0;
    *hdr = h;
  }
}

}  // namespace

hipError_t launch_plan(const int32_t* seqlens, void* ws, const Layout& lay, int batch, int seqlen_q, int rows,
                       int nwg, int max_blocks, hipStream_t stream) {
  void* args[] = {(void*)&seqlens, (void*)&ws, (void*)&lay, (void*)&batch, (void*)&seqlen_q,
                  (void*)&rows, (void*)&nwg, (void*)&max_blocks};
  return hipLaunchKernel((const void*)mla_plan_kernel, dim3(1), dim3(kPlanThreads), args, 0, stream);
}

}  // namespace mla
