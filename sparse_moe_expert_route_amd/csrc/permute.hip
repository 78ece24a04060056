// Expert permutation of the routing slots (histogram, prefix scan, stable
// rank) and the dynamic FP8 quantisation of activations gathered into expert
// order.
//
// Slots are s = t*k + j.  Rows of one expert keep ascending slot (hence
// token) order, so the result is deterministic: no atomic decides a row.
#include "moe_internal.h"
#include "fp8_rows.h"

namespace moe {

// ---------------------------------------------------------------------------
// Error bits of slot s = t*k + j holding expert id `id`: out of range, or the
// same id as an earlier slot of token t (the token's other ids are in the
// same cache line or the next).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t slot_error(const int32_t* __restrict__ ids, int s, int id, int E, int k) {
    if ((unsigned)id >= (unsigned)E) return kErrExpertIdRange;
    const int j = s % k;
    uint32_t err = 0;
    for (int i = 1; i <= j; ++i) err |= ids[s - i] == id ? kErrExpertIdDuplicate : 0u;
    return err;
}

// ---------------------------------------------------------------------------
// Pass 1: per-block expert histogram of kPermBlock slots (LDS atomics only
// count; they decide no position), and the block's error bits.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) perm_count_kernel(const int32_t* __restrict__ ids,
                                                          int32_t* __restrict__ block_counts,
                                                          uint32_t* __restrict__ block_err,
                                                          int N, int E, int k) {
    __shared__ int cnt[512];
    __shared__ uint32_t err;
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    if (threadIdx.x == 0) err = 0;
    __syncthreads();
    const int s = blockIdx.x * kPermBlock + threadIdx.x;
    if (s < N) {
        const int e = ids[s];
        if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);   // out-of-range ids are dropped
        const uint32_t bad = slot_error(ids, s, e, E, k);
        if (bad) atomicOr(&err, bad);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) block_counts[(size_t)blockIdx.x * E + e] = cnt[e];
    if (threadIdx.x == 0) block_err[blockIdx.x] = err;
}

// ---------------------------------------------------------------------------
// Pass 2 (one workgroup): for each expert, the exclusive prefix over blocks
// (block_base), then the exclusive prefix over experts of the totals
// (offsets[0..E], offsets[E] = N).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(512) perm_scan_kernel(const int32_t* __restrict__ block_counts,
                                                        int32_t* __restrict__ block_base,
                                                        int32_t* __restrict__ offsets,
                                                        const uint32_t* __restrict__ block_err,
                                                        uint32_t* __restrict__ err_word, int nblk, int E) {
    __shared__ int tot[512];
    __shared__ uint32_t err;
    const int e = threadIdx.x;
    // error word 0: the union of the blocks' error bits
    if (e == 0) err = 0;
    __syncthreads();
    uint32_t bits = 0;
    for (int b = e; b < nblk; b += 512) bits |= block_err[b];
    if (bits) atomicOr(&err, bits);
    // the exclusive prefix of expert e's column of block counts; sixteen loads
    // of a column go out together (one chain of nblk dependent loads would
    // cost a memory round trip per block: 36 us for 128 blocks)
    int run = 0;
    if (e < E) {
        int b = 0;
        for (; b + 16 <= nblk; b += 16) {
            int c[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) c[u] = block_counts[(size_t)(b + u) * E + e];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                block_base[(size_t)(b + u) * E + e] = run;
                run += c[u];
            }
        }
        for (; b < nblk; ++b) {
            const int c = block_counts[(size_t)b * E + e];
            block_base[(size_t)b * E + e] = run;
            run += c;
        }
    }
    tot[e] = (e < E) ? run : 0;
    __syncthreads();
    // Hillis-Steele inclusive scan over 512 entries
    for (int d = 1; d < 512; d <<= 1) {
        const int v = (e >= d) ? tot[e - d] : 0;
        __syncthreads();
        tot[e] += v;
        __syncthreads();
    }
    if (e < E) offsets[e] = tot[e] - run;
    if (e == E - 1) offsets[E] = tot[e];
    if (e == 0) *err_word = err;   // the scan's barriers ordered every atomicOr before this
}

// ---------------------------------------------------------------------------
// Pass 3: row of every slot = offsets[e] + block_base[b][e] + (slots of e in
// earlier waves of this block) + (slots of e in earlier lanes of this wave).
// The in-wave match mask is built from one ballot per bit of the expert id.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) perm_scatter_kernel(const int32_t* __restrict__ ids,
                                                            const int32_t* __restrict__ block_base,
                                                            const int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ sorted_token,
                                                            int32_t* __restrict__ row_of_slot,
                                                            int N, int E, int k) {
    __shared__ int wcnt[16][512];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < 16 * 512; i += blockDim.x) (&wcnt[0][0])[i] = 0;
    const int s = blockIdx.x * kPermBlock + threadIdx.x;
    const int id = s < N ? ids[s] : -1;
    const bool valid = (unsigned)id < (unsigned)E;
    const int e = valid ? id : 1023;   // 1023 never equals a real id (E <= 512)

    unsigned long long m = ~0ull;
#pragma unroll
    for (int bit = 0; bit < 10; ++bit) {
        const unsigned long long b = __ballot((e >> bit) & 1);
        m &= ((e >> bit) & 1) ? b : ~b;
    }
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(m & lt);
    __syncthreads();   // wcnt cleared
    if (valid && rank == 0) wcnt[wave][e] = __popcll(m);
    __syncthreads();
    if (!valid) {
        if (s < N) row_of_slot[s] = -1;   // an out-of-range id gets no row
        return;
    }
    int pre = 0;
    for (int w = 0; w < wave; ++w) pre += wcnt[w][e];
    const int row = offsets[e] + block_base[(size_t)blockIdx.x * E + e] + pre + rank;
    row_of_slot[s] = row;
    sorted_token[row] = s / k;
}

// ---------------------------------------------------------------------------
// Tile plan of the LDS-tiled grouped GEMMs, by one workgroup of at least 512
// threads from the expert offsets off[0..E] in LDS.  Expert e with n_e rows
// gets nt_e = ceil(n_e / rpt) m-tiles of height h_e = tile_height(n_e, nt_e)
// (its last tile holds the rest) and the token-tile class c_e = h_e / 32:
// the number of 32-row token tiles its items multiply.  Tiles are listed class
// by class (4, 3, 2, 1), experts in id order within a class and the tiles of
// one expert consecutive, so that the GEMM's workgroups move through the
// classes in one direction.  Writes tile_start[e] = first tile of expert e
// (tile_start[E] = number of tiles) and tile_info[t] = {expert, first row,
// rows, first tile of the expert} for t < max_tiles (expert -1 past the
// last tile).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int comp(const int4& v, int s) { return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w; }

__device__ void class_tile_plan(const int* __restrict__ off, int E, int rpt, int max_tiles,
                                int32_t* __restrict__ tile_start, int4* __restrict__ tile_info) {
    __shared__ int4 sc_t[512];       // inclusive prefix over experts of their tiles, per class slot 4 - c
    __shared__ int4 sc_n[512];       // ... of the experts that have tiles
    __shared__ int sstart[513], sexp[512];   // first tile and expert of the r-th expert in list order
    const int tid = threadIdx.x;
    int n = 0, nt = 0, c = 0;
    if (tid < E) {
        n = off[tid + 1] - off[tid];
        nt = (n + rpt - 1) / rpt;
        c = nt ? tile_height(n, nt) / 32 : 0;
    }
    const int slot = 4 - c;   // class 4 first
    if (tid < 512) {
        sc_t[tid] = int4{slot == 0 ? nt : 0, slot == 1 ? nt : 0, slot == 2 ? nt : 0, slot == 3 ? nt : 0};
        sc_n[tid] = int4{c && slot == 0, c && slot == 1, c && slot == 2, c && slot == 3};
    }
    __syncthreads();
    for (int d = 1; d < 512; d <<= 1) {
        int4 vt = int4{0, 0, 0, 0}, vn = int4{0, 0, 0, 0};
        if (tid < 512 && tid >= d) { vt = sc_t[tid - d]; vn = sc_n[tid - d]; }
        __syncthreads();
        if (tid < 512) {
            sc_t[tid].x += vt.x; sc_t[tid].y += vt.y; sc_t[tid].z += vt.z; sc_t[tid].w += vt.w;
            sc_n[tid].x += vn.x; sc_n[tid].y += vn.y; sc_n[tid].z += vn.z; sc_n[tid].w += vn.w;
        }
        __syncthreads();
    }
    const int4 Tt = sc_t[511], Tn = sc_n[511];
    const int total = Tt.x + Tt.y + Tt.z + Tt.w, listed = Tn.x + Tn.y + Tn.z + Tn.w;
    if (tid < E) {
        int first = 0;
        if (c) {
            int bt = 0, bn = 0;
            for (int q = 0; q < slot; ++q) { bt += comp(Tt, q); bn += comp(Tn, q); }
            first = bt + comp(sc_t[tid], slot) - nt;
            const int rank = bn + comp(sc_n[tid], slot) - 1;
            sstart[rank] = first;
            sexp[rank] = tid;
        }
        tile_start[tid] = first;
    }
    if (tid == 0) {
        tile_start[E] = total;
        sstart[listed] = total;
    }
    __syncthreads();
    for (int t = tid; t < max_tiles; t += blockDim.x) {
        int4 info = {-1, 0, 0, 0};
        if (t < total) {
            int lo = 0, hi = listed - 1;   // the last listed expert whose first tile is <= t
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (sstart[mid] <= t) lo = mid; else hi = mid - 1;
            }
            const int e = sexp[lo], t0 = sstart[lo];
            const int ne = off[e + 1] - off[e];
            const int h = tile_height(ne, (ne + rpt - 1) / rpt);
            const int row0 = off[e] + (t - t0) * h;
            info = int4{e, row0, min(h, off[e + 1] - row0), t0};
        }
        tile_info[t] = info;
    }
}

// ---------------------------------------------------------------------------
// All of the permutation for at most kPermBlock slots (decode), plus the
// tiled GEMMs' tile plan, in one workgroup: expert histogram, the two
// exclusive scans (rows and m-tiles), the stable in-block rank of every slot
// (the ballot match of perm_scatter_kernel) and the per-tile descriptors
// (max_tiles of them; 0 when the streaming GEMMs run, which need none).
// One launch instead of four.  Writes error word 0, and word 1 (= 0: its own
// offsets are valid) when it writes a tile plan.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kPermBlock) perm_small_kernel(const int32_t* __restrict__ ids,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ sorted_token,
                                                                int32_t* __restrict__ row_of_slot,
                                                                int32_t* __restrict__ tile_start,
                                                                int4* __restrict__ tile_info,
                                                                uint32_t* __restrict__ err_words,
                                                                int N, int E, int k, int rpt, int max_tiles) {
    __shared__ uint32_t err;
    __shared__ int cnt[512];
    __shared__ int scan[512];           // inclusive prefix of the rows
    __shared__ int off[513];
    __shared__ int wcnt[kPermBlock / 64][512];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < 512; i += kPermBlock) cnt[i] = 0;
    for (int i = tid; i < (kPermBlock / 64) * 512; i += kPermBlock) (&wcnt[0][0])[i] = 0;
    if (tid == 0) err = 0;
    __syncthreads();
    const int id = tid < N ? ids[tid] : -1;
    const bool valid = (unsigned)id < (unsigned)E;
    const int e = valid ? id : 1023;    // 1023 never equals a real id (E <= 512)
    if (valid) atomicAdd(&cnt[e], 1);   // counts only; no position depends on the order
    if (tid < N) {
        const uint32_t bad = slot_error(ids, tid, id, E, k);
        if (bad) atomicOr(&err, bad);
    }
    __syncthreads();
    if (tid == 0) {
        err_words[0] = err;
        if (max_tiles > 0) err_words[1] = 0;
    }
    // inclusive scan of the rows over 512 experts: Hillis-Steele on threads 0..511
    int n = 0;
    if (tid < 512) {
        n = tid < E ? cnt[tid] : 0;
        scan[tid] = n;
    }
    __syncthreads();
    for (int d = 1; d < 512; d <<= 1) {
        int v = 0;
        if (tid < 512 && tid >= d) v = scan[tid - d];
        __syncthreads();
        if (tid < 512) scan[tid] += v;
        __syncthreads();
    }
    if (tid < E) {
        off[tid] = scan[tid] - n;
        offsets[tid] = scan[tid] - n;
    }
    if (tid == E - 1) {
        off[E] = scan[tid];
        offsets[E] = scan[tid];
    }
    // stable rank of each slot among the slots of its expert
    unsigned long long m = ~0ull;
#pragma unroll
    for (int bit = 0; bit < 10; ++bit) {
        const unsigned long long b = __ballot((e >> bit) & 1);
        m &= ((e >> bit) & 1) ? b : ~b;
    }
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(m & lt);
    if (valid && rank == 0) wcnt[wave][e] = __popcll(m);
    __syncthreads();
    if (tid < N) {
        if (valid) {
            int pre = 0;
            for (int w = 0; w < wave; ++w) pre += wcnt[w][e];
            const int row = off[e] + pre + rank;
            row_of_slot[tid] = row;
            sorted_token[row] = tid / k;
        } else {
            row_of_slot[tid] = -1;   // an out-of-range id gets no row
        }
    }
    // the tiled GEMMs' tile plan (max_tiles is 0 when the streaming GEMMs run)
    if (max_tiles > 0) {
        __syncthreads();   // off[] complete
        class_tile_plan(off, E, rpt, max_tiles, tile_start, tile_info);
    }
}

hipError_t launch_perm_small(const int32_t* ids, int32_t* offsets, int32_t* sorted_token, int32_t* row_of_slot,
                             int32_t* tile_start, int4* tile_info, uint32_t* err_words, int64_t N, int E, int k,
                             int rows_per_tile, int max_tiles, hipStream_t stream) {
    hipLaunchKernelGGL(perm_small_kernel, dim3(1), dim3(kPermBlock), 0, stream, ids, offsets, sorted_token,
                       row_of_slot, tile_start, tile_info, err_words, (int)N, E, k, rows_per_tile, max_tiles);
    return hipGetLastError();
}

hipError_t launch_perm_count(const int32_t* ids, int32_t* block_counts, uint32_t* block_err, int64_t N, int E,
                             int k, hipStream_t stream) {
    const int nblk = (int)((N + kPermBlock - 1) / kPermBlock);
    hipLaunchKernelGGL(perm_count_kernel, dim3(nblk), dim3(kPermBlock), 0, stream, ids, block_counts, block_err,
                       (int)N, E, k);
    return hipGetLastError();
}

hipError_t launch_perm_scan(const int32_t* block_counts, int32_t* block_base, int32_t* offsets,
                            const uint32_t* block_err, uint32_t* err_word, int64_t N, int E, hipStream_t stream) {
    const int nblk = (int)((N + kPermBlock - 1) / kPermBlock);
    hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(512), 0, stream, block_counts, block_base, offsets, block_err,
                       err_word, nblk, E);
    return hipGetLastError();
}

hipError_t launch_perm_scatter(const int32_t* ids, const int32_t* block_base, const int32_t* offsets,
                               int32_t* sorted_token, int32_t* row_of_slot, int64_t N, int E, int k,
                               hipStream_t stream) {
    const int nblk = (int)((N + kPermBlock - 1) / kPermBlock);
    hipLaunchKernelGGL(perm_scatter_kernel, dim3(nblk), dim3(kPermBlock), 0, stream, ids, block_base, offsets,
                       sorted_token, row_of_slot, (int)N, E, k);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Quantise + gather: row r of the output is FP8(x[sorted_token[r]]), or
// FP8(x[r]) without sorted_token (the gather then happens in GEMM-1).  The
// row quantiser itself is in fp8_rows.h.
// ---------------------------------------------------------------------------
template <bool F32S>
__global__ void __launch_bounds__(256) quant_gather_kernel(const uint16_t* __restrict__ x,
                                                           const int32_t* __restrict__ sorted_token,
                                                           uint8_t* __restrict__ xq, void* __restrict__ xs,
                                                           int N, int H, int T) {
    for (int r = blockIdx.x; r < N; r += gridDim.x) {
        // (no sorted_token: quantise the tokens in their own order)
        const int t = sorted_token ? min(max(sorted_token[r], 0), T - 1) : r;   // rows left unfilled by invalid ids stay in bounds
        quantise_row<F32S>(x + (size_t)t * H, xq, xs, r, H);
    }
}

hipError_t launch_quant_gather(const uint16_t* x, const int32_t* sorted_token, uint8_t* xq, void* xs,
                               int64_t N, int H, int64_t T, int f32_scales, hipStream_t stream) {
    const int grid = (int)(N < 65536 ? N : 65536);
    if (f32_scales)
        hipLaunchKernelGGL(quant_gather_kernel<true>, dim3(grid), dim3(256), 0, stream, x, sorted_token, xq, xs,
                           (int)N, H, (int)T);
    else
        hipLaunchKernelGGL(quant_gather_kernel<false>, dim3(grid), dim3(256), 0, stream, x, sorted_token, xq, xs,
                           (int)N, H, (int)T);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Tile plan of the grouped GEMMs from caller-given offsets (class_tile_plan).
// The offsets come from the caller on the staged entry points, so they are
// checked first: unless 0 = o[0] <= ... <= o[E] = N the plan is empty (the
// GEMMs do nothing) and error word 1 says why.  Valid offsets give at most
// ceil(N / rpt) + E = max_tiles tiles.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(512) tile_plan_kernel(const int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ tile_start, int4* __restrict__ tile_info,
                                                        uint32_t* __restrict__ err_word, int E, int rpt,
                                                        int max_tiles, int N) {
    __shared__ int off[513];
    const int e = threadIdx.x;
    const int o0 = (e < E) ? offsets[e] : 0, o1 = (e < E) ? offsets[e + 1] : 0;
    bool bad = o0 > o1 || (e == 0 && o0 != 0) || (e == E - 1 && o1 != N);
    bad = __syncthreads_or(bad);
    if (e == 0) *err_word = bad ? kErrExpertOffsets : 0u;
    // invalid offsets: every expert empty, an empty plan
    if (e < E) off[e] = bad ? 0 : o0;
    if (e == E - 1) off[E] = bad ? 0 : o1;
    __syncthreads();
    class_tile_plan(off, E, rpt, max_tiles, tile_start, tile_info);
}

hipError_t launch_tile_plan(const int32_t* offsets, int32_t* tile_start, int4* tile_info, uint32_t* err_word, int E,
                            int rows_per_tile, int max_tiles, int64_t N, hipStream_t stream) {
    hipLaunchKernelGGL(tile_plan_kernel, dim3(1), dim3(512), 0, stream, offsets, tile_start, tile_info, err_word, E,
                       rows_per_tile, max_tiles, (int)N);
    return hipGetLastError();
}

}  // namespace moe
