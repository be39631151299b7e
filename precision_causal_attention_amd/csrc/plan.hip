// GPU-built tile lists, expensive items first (FLAMIA paper, Section 3.6.2
// and Appendix B.6): built on the device in one single-workgroup launch, no
// host synchronization.
//
// A document of L tokens has n = ceil(L/128) tiles of 128 tokens, anchored at
// its first token.
//   query-major (forward, dQ): query tile t attends t+1 key tiles  -> cost t + 1
//   key-major (dK/dV)        : key tile t meets n - t query tiles  -> cost n - t
// Both give every document the costs 1..n.  Two orders, both with the
// expensive items first (the hardware dispatches workgroups in index order,
// so the expensive items start first and the cheap ones fill in at the end):
//   document-major: documents by decreasing tile count, and within a
//   document its tiles by decreasing cost, so the items that run at the same
//   time on an XCD mostly belong to one document and share its K/V (query
//   major) or Q/dO rows (key major) in that XCD's L2;
//   cost-major: all tiles by decreasing cost, documents interleaved.
// The query-major list is document-major; the key-major one is document-major
// when the caller asks for it (the attention library does at both head
// dimensions), else cost-major.  A document-major list ends with every
// document's cheapest tiles (query-major: the first, key-major: the last
// two), by decreasing cost, which fill in the tail as in the cost-major order.  Beyond
// kPrefixLds documents both lists are cost-major.  Sorting is a counting sort on the small integer tile count
// or cost instead of a comparison sort.  Within one class the order is
// whatever the atomics give; it does not change any result.
// Work item (tile, head) is decoded by the attention kernels from the
// workgroup index, heads innermost.
//
// A malformed cu_seqlens (cu[0] != 0, a decreasing pair, a boundary outside
// [0, ttot], or cu[ndocs] != ttot) yields no tile at all, so the attention
// kernels do no work, and the caller's status word (when given) gets the
// reason: bit 0 cu[0] != 0, bit 1 a decreasing pair, bit 2 a boundary outside
// [0, ttot] or cu[ndocs] != ttot; 0 for a well-formed array.
//
// ctrl layout (int32): [0] number of tiles, [1] 1 if the backward's dS store
// holds this call's blocks (capacity given and not exceeded), else 0, [2] the
// work-queue counter of the persistent key-major pass at d = 128 (zeroed here,
// by every call, before that pass runs), [32 .. 47] 64 zero bytes that the
// attention kernels' staged loads read for rows past a document's end
// (written by every call).  cu_seqlens (up to kPrefixLds
// documents), the tile prefix of the documents, their document-major slots
// and the placement cursors live in LDS.  The dS block offsets of the
// documents go to dboff.
#include "device.h"
#include "kernels.h"

namespace {
// Tiles of cost <= kTail* go to the end of the document-major lists, where
// they fill in the tail (16 x 1024-token documents: forward 73.6 -> 68.3 us,
// dQ pass 110.8 -> 104.4 us with 1 for the query-major list; 2 was no
// better there and 0.4% slower on the 4 x 8192 GQA call).  The key-major
// list moves the last two key tiles of every document (with 1, on the
// 4 x 8192 GQA call, the first tiles of the shortest documents started last
// and ended the launch, per-workgroup timestamps showed): dK/dV 407 -> 397
// us against 1 (3 and 5: 399-402 us), no change on the d = 128 workloads.
constexpr int kTailQ = 1;
constexpr int kTailK = 2;
}  // namespace

namespace flamia {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kPrefixLds = 4096;          // documents whose tile prefix is kept in LDS

// Inclusive scans of two values per thread over the block at once: a shuffle
// scan in each wave, then the wave totals (integer sums: the result does not
// depend on the order).  va, vb become this thread's inclusive prefixes, ta,
// tb the block's sums.  Two barriers; wa and wb are free again on return.
template <typename A, typename B>
__device__ void block_incl_scan2(A& va, B& vb, A* wa, B* wb, A& ta, B& tb) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const A x = __shfl_up(va, off);
        const B y = __shfl_up(vb, off);
        if (lane >= off) {
            va += x;
            vb += y;
        }
    }
    if (lane == 63) {
        wa[w] = va;
        wb[w] = vb;
    }
    __syncthreads();
    A ba = 0, sa = 0;
    B bb = 0, sb = 0;
#pragma unroll
    for (int i = 0; i < kPlanWaves; ++i) {
        const A x = wa[i];
        const B y = wb[i];
        if (i < w) {
            ba += x;
            bb += y;
        }
        sa += x;
        sb += y;
    }
    __syncthreads();
    ta = sa;
    tb = sb;
    va += ba;
    vb += bb;
}

// In-place inclusive suffix scans of a[0..n) and b[0..n) in LDS (sums from the
// end).  Each thread owns one contiguous chunk.
__device__ void block_suffix_scan2(int* a, int* b, int n, int* wa, int* wb) {
    const int tid = threadIdx.x;
    const int chunk = (n + kPlanThreads - 1) / kPlanThreads;
    const int lo = tid * chunk, hi = min(lo + chunk, n);
    int sa = 0, sb = 0;
    for (int i = lo; i < hi; ++i) {
        sa += a[n - 1 - i];
        sb += b[n - 1 - i];
    }
    int ta, tb;
    int ra = sa, rb = sb;
    block_incl_scan2(ra, rb, wa, wb, ta, tb);
    ra -= sa;
    rb -= sb;
    for (int i = lo; i < hi; ++i) {
        ra += a[n - 1 - i];
        rb += b[n - 1 - i];
        a[n - 1 - i] = ra;
        b[n - 1 - i] = rb;
    }
    __syncthreads();
}

__global__ void __launch_bounds__(kPlanThreads)
plan_kernel(const int32_t* __restrict__ cu, int ndocs, int ttot, int32_t* __restrict__ cu_status,
            int max_cost, int32_t* __restrict__ tiles_prefix,
            int32_t* __restrict__ ctrl, long max_tiles, int4* __restrict__ tiles_q, int4* __restrict__ tiles_k,
            int key_docmajor, int32_t* __restrict__ dboff, long ds_blocks) {
    extern __shared__ int smem[];
    const int C1 = max_cost + 1;
    int* hist = smem;                          // C1: tile counts by cost class
    // C1 each: placement cursors of the cost-major lists; with the LDS prefix
    // table curq first holds the tiles of the documents with at least c tiles
    // and curk the document cursors by tile count (document-major order)
    int* curq = smem + C1;
    int* curk = smem + 2 * C1;
    __shared__ int wsum[kPlanWaves];
    __shared__ int wsum2[kPlanWaves];
    __shared__ long lwsum[kPlanWaves];
    __shared__ int lpref[kPrefixLds];          // tile prefix of the documents (ndocs < kPrefixLds)
    __shared__ int ldbase[kPrefixLds];         // first slot of each document, document-major
    __shared__ int lcu[kPrefixLds + 1];        // cu_seqlens (ndocs < kPrefixLds)
    __shared__ int bad_all;
    const int tid = threadIdx.x;
    const bool lds_pref = ndocs < kPrefixLds;
    if (tid < 16) ctrl[32 + tid] = 0;
    // cu_seqlens is read from global memory once when it fits in LDS
    if (lds_pref)
        for (int d = tid; d <= ndocs; d += kPlanThreads) lcu[d] = cu[d];
    if (tid == 0) bad_all = 0;
    __syncthreads();
    const int32_t* cux = lds_pref ? lcu : cu;
    // ---- the packed layout's preconditions (Section 3.6.1)
    int bad = 0;
    for (int d = tid; d < ndocs; d += kPlanThreads) {
        const int a0 = cux[d], a1 = cux[d + 1];
        if (a1 < a0) bad |= 2;
        if (a0 < 0 || a1 > ttot) bad |= 4;
    }
    if (tid == 0) {
        if (cux[0] != 0) bad |= 1;
        if (cux[ndocs] != ttot) bad |= 4;
    }
    if (bad) atomicOr(&bad_all, bad);
    __syncthreads();
    if (tid == 0 && cu_status) *cu_status = bad_all;
    if (bad_all) {
        if (tid == 0) ctrl[0] = ctrl[1] = ctrl[2] = 0;
        return;
    }
    for (int c = tid; c < C1; c += kPlanThreads) hist[c] = curq[c] = curk[c] = 0;
    __syncthreads();
    for (int d = tid; d < ndocs; d += kPlanThreads) {
        const int L = cux[d + 1] - cux[d];
        const int n = min((L + kTile - 1) / kTile, max_cost);
        if (n > 0) atomicAdd(&hist[n], 1);
    }
    __syncthreads();
    // With cnt[c] = #docs with n == c, one pass of suffix sums gives
    //   A[c] = #docs with n >= c = number of tiles of cost c (c >= 1), and
    //   above[c] = sum over n >= c of n cnt[n] = tiles of the documents with
    //   at least c tiles (document-major slots);
    // the number of tiles of cost >= c (cost-major slots: the class of cost c
    // starts at hist[c + 1]) is then sum over n >= c of cnt[n] (n - c + 1) =
    // above[c] - (c - 1) A[c], and hist[1] is the total.
    int* above = curq;
    for (int c = tid; c < C1; c += kPlanThreads) above[c] = c * hist[c];
    __syncthreads();
    block_suffix_scan2(hist, above, C1, wsum, wsum2);
    for (int c = tid; c < C1; c += kPlanThreads) hist[c] = above[c] - (c - 1) * hist[c];
    // the cost-major query list places with the cursors curq (document-major
    // keeps `above`)
    if (!lds_pref)
        for (int c = tid; c < C1; c += kPlanThreads) curq[c] = 0;
    __syncthreads();
    const int total = C1 > 1 ? (int)min((long)hist[1], max_tiles) : 0;
    if (tid == 0) {
        ctrl[0] = total;
        ctrl[2] = 0;
    }
    // exclusive prefix of tile counts over documents and, with a dS store,
    // of their causal 32x32 blocks (nb (nb + 1) / 2 for nb = ceil(L / 32):
    // each document's first block), in one scan
    {
        const int chunk = (ndocs + kPlanThreads - 1) / kPlanThreads;
        const int lo = tid * chunk, hi = min(lo + chunk, ndocs);
        auto tiles_of = [&](int d) { return (cux[d + 1] - cux[d] + kTile - 1) / kTile; };
        auto blocks_of = [&](int d) -> long {
            const long nb = (cux[d + 1] - cux[d] + kBlock - 1) / kBlock;
            return nb * (nb + 1) / 2;
        };
        int sum = 0;
        long bsum = 0;
        for (int d = lo; d < hi; ++d) {
            sum += tiles_of(d);
            if (dboff) bsum += blocks_of(d);
        }
        int all;
        long total_blocks;
        int run = sum;
        long brun = bsum;
        block_incl_scan2(run, brun, wsum, lwsum, all, total_blocks);
        run -= sum;
        brun -= bsum;
        const bool fits = dboff && ds_blocks > 0 && total_blocks <= ds_blocks;
        for (int d = lo; d < hi; ++d) {
            tiles_prefix[d] = run;
            if (lds_pref) lpref[d] = run;
            run += tiles_of(d);
            if (dboff) {
                dboff[d] = fits ? (int32_t)brun : 0;
                brun += blocks_of(d);
            }
        }
        if (tid == 0) {
            tiles_prefix[ndocs] = all;
            if (lds_pref) lpref[ndocs] = all;
            // 1 if the backward's dS store holds this call's blocks
            ctrl[1] = fits ? 1 : 0;
        }
    }
    // the prefix table (LDS, or global beyond kPrefixLds documents, which then
    // must have reached L2) is complete for every thread
    if (!lds_pref) __threadfence();
    __syncthreads();
    // document-major: each document's first slot, after the documents with
    // more tiles
    if (lds_pref) {
        int* curd = curk;
        for (int d = tid; d < ndocs; d += kPlanThreads) {
            const int n = lpref[d + 1] - lpref[d];
            const int c = min(n, max_cost);
            if (n > 0) ldbase[d] = (c + 1 < C1 ? above[c + 1] : 0) + atomicAdd(&curd[c], n);
        }
        __syncthreads();
        for (int c = tid; c < C1; c += kPlanThreads) curk[c] = 0;
        __syncthreads();
    }
    // Document-major slot of the tile of cost `cost` (1..n) of document doc
    // (n tiles) when the tiles of cost <= T go to the end of the list: the
    // list is document-major over the tiles of cost > T, then the tiles of
    // cost T, T - 1, ..., 1, each class in document order; those short
    // items fill in the tail, as in the cost-major order.  A[j] (documents
    // with at least j tiles) follows from hist[j] = above[j] - (j - 1) A[j];
    // a document's rank (documents placed before it) is A[n + 1] plus its
    // place in its class (cursor offset / n); the documents before it have
    // at least n > T tiles, so its first main slot is ldbase - T rank.
    auto docs_with = [&](int j) -> int {
        if (j == 1) return hist[1] - (C1 > 2 ? hist[2] : 0);
        return j < C1 ? (above[j] - hist[j]) / (j - 1) : 0;
    };
    auto dm_slot = [&](int doc, int n, int cost, int T) -> int {
        const int c = min(n, max_cost);
        const int rank = docs_with(c + 1) + (ldbase[doc] - (c + 1 < C1 ? above[c + 1] : 0)) / n;
        if (cost > T) return ldbase[doc] - T * rank + (n - cost);
        int start = total;
        for (int j = 1; j <= cost; ++j) start -= docs_with(j);
        return start + rank;
    };
    // tile p, the t-th of the n tiles of document doc, whose first tile is pre
    const bool kdoc = lds_pref && key_docmajor;
    auto place = [&](int p, int doc, int pre, int next) {
        const int t = p - pre;
        const int n = next - pre;
        const int ds = cux[doc], de = cux[doc + 1];
        const int4 tile = make_int4(ds + kTile * t, ds, de, doc);
        {
            const int cost = t + 1;
            const int slot = lds_pref ? dm_slot(doc, n, cost, kTailQ)
                                      : (cost + 1 < C1 ? hist[cost + 1] : 0) + atomicAdd(&curq[cost], 1);
            if (slot < max_tiles) tiles_q[slot] = tile;
        }
        if (tiles_k) {
            const int cost = n - t;
            const int slot = kdoc ? dm_slot(doc, n, cost, kTailK)
                                  : (cost + 1 < C1 ? hist[cost + 1] : 0) + atomicAdd(&curk[cost], 1);
            if (slot < max_tiles) tiles_k[slot] = tile;
        }
    };
    if (lds_pref) {
        for (int p = tid; p < total; p += kPlanThreads) {
            // the document of tile p: binary search of the LDS prefix
            int lo = 0, hi = ndocs - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (lpref[mid] <= p) lo = mid; else hi = mid - 1;
            }
            place(p, lo, lpref[lo], lpref[lo + 1]);
        }
    } else {
        for (int p = tid; p < total; p += kPlanThreads) {
            const int doc = find_doc(tiles_prefix, ndocs, p);
            place(p, doc, tiles_prefix[doc], tiles_prefix[doc + 1]);
        }
    }
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t st) {
    const size_t smem = sizeof(int) * 3 * ((size_t)a.max_cost + 1);
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), smem, st, a.cu, a.ndocs, a.ttot, a.cu_status,
                       a.max_cost, a.tiles_prefix, a.ctrl, a.max_tiles, a.tiles_q, a.tiles_k, a.key_docmajor,
                       a.dboff, a.ds_blocks);
    return hipGetLastError();
}

}  // namespace flamia
