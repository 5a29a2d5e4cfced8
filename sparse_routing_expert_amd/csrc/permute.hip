// moe_permute kernels: expert histogram, exclusive scan, stable ranking and the row scatter that
// packs every expert's tokens into one contiguous buffer ("Router Optimization Techniques",
// What Most Articles Miss 2), each expert's rows in ascending token order -- the order of the
// per-expert nonzero() in "Fine-tuning and serving MoE models", How an MoE layer actually works.
//
// Assignments a = t*k + j are cut into tiles of kPermTile. perm_local ranks every assignment inside
// its tile with wave ballots (stable, no atomics) and writes the tile's per-expert counts;
// perm_scan turns the [tile][expert] counts into expert offsets and per-tile rank bases (small
// routers skip it: the scatter forms both from the counts); perm_place_scatter gives each
// assignment its row, drops the ones ranked at or past an expert capacity ("Router Optimization
// Techniques", Why It Matters 3 and FAQ 6), and reads each token row once to write its kept copies
// with 128-bit stores. Batches of at most 4096 assignments take one block for the whole index stage
// (perm_index_small) and the plain scatter.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

// One block of 1024 threads: J = 1024 / Ep threads per expert (Ep = E rounded up to a power of two),
// thread (e, j) owning the contiguous tile range [j * C, (j + 1) * C), C = ceil(ntiles / J). Each
// thread sums its range (loads issued 8 at a time), the J range sums of an expert are scanned in
// LDS, and each thread then writes tile_base[tile][e] = assignments to e in earlier tiles over its
// range. offsets = exclusive scan of the rows each expert keeps (min(count, capacity) with a
// capacity).
__global__ __launch_bounds__(1024) void perm_scan_kernel(const int32_t* __restrict__ tile_counts, int ntiles,
                                                         int E, int Ep, int capacity, int32_t* __restrict__ tile_base,
                                                         int32_t* __restrict__ offsets) {
    __shared__ int s_rng[1024];
    __shared__ int s_wave[17];
    const int J = 1024 / Ep;
    const int e = threadIdx.x / J, j = threadIdx.x % J;
    const int C = (ntiles + J - 1) / J;
    const int tb = j * C, te = tb + C < ntiles ? tb + C : ntiles;
    int sum = 0;
    if (e < E) {
        int tile = tb;
        for (; tile + 8 <= te; tile += 8) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = tile_counts[(int64_t)(tile + u) * E + e];
#pragma unroll
            for (int u = 0; u < 8; ++u) sum += v[u];
        }
        for (; tile < te; ++tile) sum += tile_counts[(int64_t)tile * E + e];
    }
    s_rng[threadIdx.x] = sum;
    __syncthreads();
    // expert totals (thread e < Ep sums its expert's J ranges), scanned over experts
    int tot = 0;
    if (threadIdx.x < Ep)
        for (int jj = 0; jj < J; ++jj) tot += s_rng[threadIdx.x * J + jj];
    const int kept = threadIdx.x < E ? (capacity > 0 && tot > capacity ? capacity : tot) : 0;
    int total;
    const int start = block1024_excl_scan(kept, s_wave, &total);
    if (threadIdx.x < E) offsets[threadIdx.x] = start;
    if (threadIdx.x == 0) offsets[E] = total;
    if (e >= E) return;
    int run = 0;
    for (int jj = 0; jj < j; ++jj) run += s_rng[e * J + jj];
    int tile = tb;
    for (; tile + 8 <= te; tile += 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = tile_counts[(int64_t)(tile + u) * E + e];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            tile_base[(int64_t)(tile + u) * E + e] = run;
            run += v[u];
        }
    }
    for (; tile < te; ++tile) {
        tile_base[(int64_t)tile * E + e] = run;
        run += tile_counts[(int64_t)tile * E + e];
    }
}

// One wave per token: read the row once, store it at its k destinations (16-byte vectors, up to
// 8 per lane loaded before any store so a row is one memory round trip); dropped slots (-1) are
// skipped. Loads and stores are non-temporal: each byte is touched once here.
__global__ __launch_bounds__(256) void perm_scatter_kernel(const uint8_t* __restrict__ x,
                                                           const int32_t* __restrict__ inv_pos, int64_t T,
                                                           int row_bytes, int k, uint8_t* __restrict__ x_perm) {
    constexpr int U = 8;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= T) return;
    const int mypos = lane < k ? inv_pos[t * k + lane] : 0;
    const int nchunks = row_bytes / 16;
    const uint8_t* src = x + t * row_bytes;
    for (int c0 = lane; c0 < nchunks; c0 += 64 * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (c0 + 64 * u < nchunks) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (int64_t)(c0 + 64 * u) * 16));
        for (int j = 0; j < k; ++j) {
            const int p = __builtin_amdgcn_readlane(mypos, j);
            if (p < 0) continue;
            uint8_t* dst = x_perm + (int64_t)p * row_bytes;
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (c0 + 64 * u < nchunks)
                    __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(dst + (int64_t)(c0 + 64 * u) * 16));
        }
    }
}

// Tile histogram and stable in-tile ranks in one pass. The tile is processed as 16 chunks of 64
// consecutive assignments (chunk c = iteration * 4 + wave). Inside a chunk, lanes holding the same
// expert are found by intersecting ballots over the bits of the expert id; the lane's rank among them
// is the popcount below it, and the chunk's count per expert goes to LDS. An assignment's in-tile rank
// (earlier assignments of the tile to the same expert) goes to local_rank[a], the tile's per-expert
// totals to tile_counts. perm_place_scatter_kernel turns the rank into the row.
__global__ __launch_bounds__(256) void perm_local_kernel(const int32_t* __restrict__ idx, int64_t A, int E,
                                                         int nbits, int32_t* __restrict__ tile_counts,
                                                         int32_t* __restrict__ local_rank) {
    constexpr int ITERS = kPermTile / 256;
    constexpr int CHUNKS = kPermTile / 64;
    extern __shared__ int cnt[];  // [CHUNKS][E]
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < CHUNKS * E; i += 256) cnt[i] = 0;
    __syncthreads();
    const int64_t a0 = (int64_t)blockIdx.x * kPermTile;
    const uint64_t below = (1ull << lane) - 1ull;
    int rank[ITERS], ev[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int64_t a = a0 + it * 256 + threadIdx.x;
        ev[it] = a < A ? idx[a] : E;  // E never equals a real expert id
    }
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int e = ev[it];
        uint64_t m = ~0ull;
        for (int b = 0; b < nbits; ++b) {
            const int bit = (e >> b) & 1;
            const uint64_t bb = __ballot(bit);
            m &= bit ? bb : ~bb;
        }
        const int rk = __popcll(m & below);
        if (e < E && rk == 0) cnt[(it * 4 + wave) * E + e] = __popcll(m);
        rank[it] = rk;
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int64_t a = a0 + it * 256 + threadIdx.x;
        if (a >= A) continue;
        const int e = ev[it];
        const int c = it * 4 + wave;
        int r = rank[it];
        for (int c2 = 0; c2 < c; ++c2) r += cnt[c2 * E + e];
        local_rank[a] = r;
    }
    for (int e = threadIdx.x; e < E; e += 256) {
        int sum = 0;
#pragma unroll
        for (int c = 0; c < CHUNKS; ++c) sum += cnt[c * E + e];
        tile_counts[(int64_t)blockIdx.x * E + e] = sum;
    }
}

// perm_scatter_kernel that first places its token's assignments: row = offsets[e] + (assignments to e
// in earlier tiles) + in-tile rank, or dropped (-1) at or past the capacity; it writes inv_pos (over
// the in-tile rank it held) and sorted_token, then copies the row. FOLD (E <= kPermFoldExperts and at
// most kPermFoldTiles tiles): the block forms the expert offsets and its tiles' bases itself from the
// tile counts, so no scan launch runs, and block 0 writes offsets. Otherwise perm_scan_kernel's
// tile_base and offsets are read.
template <bool FOLD>
__global__ __launch_bounds__(256) void perm_place_scatter_kernel(
    const uint8_t* __restrict__ x, const int32_t* __restrict__ idx, const int32_t* __restrict__ tile_counts,
    const int32_t* __restrict__ tile_base, int32_t* __restrict__ offsets, int ntiles, int E, int capacity, int64_t T,
    int row_bytes, int k, int32_t* __restrict__ inv_pos, int32_t* __restrict__ sorted_token,
    uint8_t* __restrict__ x_perm) {
    constexpr int U = 8;
    __shared__ int s_kept[FOLD ? kPermFoldExperts : 1];
    __shared__ int s_off[FOLD ? kPermFoldExperts : 1];
    __shared__ int s_pre[2][FOLD ? kPermFoldExperts : 1];
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    // the block's 4 k assignments span at most two tiles (4 k <= kPermTile)
    const int64_t tile_lo = (int64_t)blockIdx.x * 4 * k / kPermTile;
    if (FOLD) {
        const int e = threadIdx.x;
        if (e < E) {
            int tot = 0, pre = 0, at_lo = 0;
            for (int t0 = 0; t0 < ntiles; t0 += 8) {  // 8 loads in flight
                int c[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) c[u] = t0 + u < ntiles ? tile_counts[(t0 + u) * E + e] : 0;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    pre += t0 + u < tile_lo ? c[u] : 0;
                    at_lo = t0 + u == tile_lo ? c[u] : at_lo;
                    tot += c[u];
                }
            }
            s_pre[0][e] = pre;
            s_pre[1][e] = pre + at_lo;
            s_kept[e] = capacity > 0 && tot > capacity ? capacity : tot;
        }
        __syncthreads();
        if (e < E) {
            int o = 0;
            for (int e2 = 0; e2 < e; ++e2) o += s_kept[e2];
            s_off[e] = o;
            if (blockIdx.x == 0) {
                offsets[e] = o;
                if (e == E - 1) offsets[E] = o + s_kept[e];
            }
        }
        __syncthreads();
    }
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= T) return;
    int mypos = 0;
    if (lane < k) {
        const int64_t a = t * k + lane;
        const int e = idx[a];
        const int64_t tile = a / kPermTile;
        const int r = (FOLD ? s_pre[tile - tile_lo][e] : tile_base[tile * E + e]) + inv_pos[a];
        mypos = capacity > 0 && r >= capacity ? -1 : (FOLD ? s_off[e] : offsets[e]) + r;
        inv_pos[a] = mypos;
        if (mypos >= 0) sorted_token[mypos] = (int32_t)t;
    }
    const int nchunks = row_bytes / 16;
    const uint8_t* src = x + t * row_bytes;
    for (int c0 = lane; c0 < nchunks; c0 += 64 * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (c0 + 64 * u < nchunks) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (int64_t)(c0 + 64 * u) * 16));
        for (int j = 0; j < k; ++j) {
            const int p = __builtin_amdgcn_readlane(mypos, j);
            if (p < 0) continue;
            uint8_t* dst = x_perm + (int64_t)p * row_bytes;
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (c0 + 64 * u < nchunks)
                    __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(dst + (int64_t)(c0 + 64 * u) * 16));
        }
    }
}

// The placing step of perm_place_scatter_kernel without the row copy (x_perm == NULL, the forward's
// form): one thread per assignment instead of one wave per token, so a block of 256 consecutive
// assignments (inside one tile, as 256 divides kPermTile) forms the expert offsets and its tile's
// bases once for 256 assignments instead of for 4 tokens. Same rows, same dropping rule.
template <bool FOLD>
__global__ __launch_bounds__(256) void perm_place_kernel(const int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ tile_counts,
                                                         const int32_t* __restrict__ tile_base,
                                                         int32_t* __restrict__ offsets, int ntiles, int E,
                                                         int capacity, int64_t A, int k,
                                                         int32_t* __restrict__ inv_pos,
                                                         int32_t* __restrict__ sorted_token) {
    static_assert(kPermTile % 256 == 0, "a block's assignments lie in one tile");
    __shared__ int s_kept[FOLD ? kPermFoldExperts : 1];
    __shared__ int s_off[FOLD ? kPermFoldExperts : 1];
    __shared__ int s_pre[FOLD ? kPermFoldExperts : 1];
    const int64_t a0 = (int64_t)blockIdx.x * 256;
    const int64_t tile = a0 / kPermTile;
    if (FOLD) {
        const int e = threadIdx.x;
        if (e < E) {
            int tot = 0, pre = 0;
            for (int t0 = 0; t0 < ntiles; t0 += 8) {  // 8 loads in flight
                int c[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) c[u] = t0 + u < ntiles ? tile_counts[(t0 + u) * E + e] : 0;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    pre += t0 + u < tile ? c[u] : 0;
                    tot += c[u];
                }
            }
            s_pre[e] = pre;
            s_kept[e] = capacity > 0 && tot > capacity ? capacity : tot;
        }
        __syncthreads();
        if (e < E) {
            int o = 0;
            for (int e2 = 0; e2 < e; ++e2) o += s_kept[e2];
            s_off[e] = o;
            if (blockIdx.x == 0) {
                offsets[e] = o;
                if (e == E - 1) offsets[E] = o + s_kept[e];
            }
        }
        __syncthreads();
    }
    const int64_t a = a0 + threadIdx.x;
    if (a >= A) return;
    const int e = idx[a];
    const int r = (FOLD ? s_pre[e] : tile_base[tile * E + e]) + inv_pos[a];
    const int pos = capacity > 0 && r >= capacity ? -1 : (FOLD ? s_off[e] : offsets[e]) + r;
    inv_pos[a] = pos;
    if (pos >= 0) sorted_token[pos] = (int32_t)(a / k);
}

// The whole index stage in one block of 1024 threads, for layers whose per-chunk expert counts fit
// in LDS (chunks of 64 assignments, ceil(A / 64) * E <= kPermSmallCounts). The same positions as
// the tiled kernels (stable in (t, j) order, dropped past the capacity), in one launch:
//  1. wave w loads the expert ids of chunks w, w + 16, ... (at most kPermSmallChunksPerWave) at
//     once, matches each chunk's assignments by ballots over the id bits and stores the chunk's
//     count per expert (no atomics);
//  2. per expert, J = min(64, 1024 / Ep) lanes of one wave each own a contiguous range of chunks;
//     the range sums are scanned across those lanes by shuffles, and each lane rewrites its chunks'
//     counts as exclusive bases (assignments to e in earlier chunks); the expert totals (capped at
//     the capacity) are scanned over experts into offsets;
//  3. the chunks are matched again from the held ids, and each assignment gets row
//     offsets[e] + base + rank.
__global__ __launch_bounds__(1024) void perm_index_small_kernel(const int32_t* __restrict__ idx, int64_t A, int E,
                                                                int k, int nbits, int Ep, int capacity,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ inv_pos,
                                                                int32_t* __restrict__ sorted_token) {
    extern __shared__ int cnt[];  // [nch][E]
    __shared__ int s_tot[1024];
    __shared__ int s_off[1025];
    __shared__ int s_wave[17];
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int nch = (int)((A + 63) / 64);
    for (int i = threadIdx.x; i < nch * E; i += 1024) cnt[i] = 0;
    __syncthreads();
    const uint64_t below = (1ull << lane) - 1ull;
    // every expert id of the wave's chunks, loaded at once (chunk wave + 16 i in ev[i]); E marks
    // positions past A and never equals a real expert id
    int ev[kPermSmallChunksPerWave];
#pragma unroll
    for (int i = 0; i < kPermSmallChunksPerWave; ++i) {
        const int64_t a = (int64_t)(wave + 16 * i) * 64 + lane;
        ev[i] = a < A ? idx[a] : E;
    }
    auto match = [&](int e, int& rk) -> uint64_t {
        uint64_t m = ~0ull;
        for (int b = 0; b < nbits; ++b) {
            const int bit = (e >> b) & 1;
            const uint64_t bb = __ballot(bit);
            m &= bit ? bb : ~bb;
        }
        rk = __popcll(m & below);
        return m;
    };
#pragma unroll
    for (int i = 0; i < kPermSmallChunksPerWave; ++i) {
        const int c = wave + 16 * i;
        if (c >= nch) break;  // uniform per wave
        int rk;
        const uint64_t m = match(ev[i], rk);
        if (ev[i] < E && rk == 0) cnt[c * E + ev[i]] = __popcll(m);
    }
    __syncthreads();
    // per-expert exclusive bases over chunks
    const int J = 1024 / Ep < 64 ? 1024 / Ep : 64;
    const int e = threadIdx.x / J, j = threadIdx.x % J;
    const int C = (nch + J - 1) / J;
    const int cb = j * C < nch ? j * C : nch, ce = cb + C < nch ? cb + C : nch;
    int sum = 0;
    if (e < E)
        for (int c = cb; c < ce; ++c) sum += cnt[c * E + e];
    int inc = sum;  // inclusive scan over the J lanes of this expert (one segment of a wave)
    for (int o = 1; o < J; o <<= 1) {
        const int n = __shfl_up(inc, o, J);
        if (j >= o) inc += n;
    }
    if (e < E) {
        int run = inc - sum;
        for (int c = cb; c < ce; ++c) {
            const int v = cnt[c * E + e];
            cnt[c * E + e] = run;
            run += v;
        }
        if (j == J - 1) s_tot[e] = inc;
    }
    __syncthreads();
    const int tot = threadIdx.x < E ? s_tot[threadIdx.x] : 0;
    const int kept = capacity > 0 && tot > capacity ? capacity : tot;
    int total;
    const int start = block1024_excl_scan(kept, s_wave, &total);
    if (threadIdx.x < E) {
        offsets[threadIdx.x] = start;
        s_off[threadIdx.x] = start;
    }
    if (threadIdx.x == 0) offsets[E] = total;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPermSmallChunksPerWave; ++i) {
        const int c = wave + 16 * i;
        if (c >= nch) break;  // uniform per wave
        const int64_t a = (int64_t)c * 64 + lane;
        const int ea = ev[i];
        int rk;
        match(ea, rk);
        if (a >= A) continue;
        const int r = cnt[c * E + ea] + rk;
        if (capacity > 0 && r >= capacity) {
            inv_pos[a] = -1;
            continue;
        }
        const int pos = s_off[ea] + r;
        inv_pos[a] = pos;
        sorted_token[pos] = (int32_t)(a / k);
    }
}

bool perm_index_small_ok(int64_t A, int E) {
    // where the tiled path folds its scan into the scatter (two launches, like this one) it is the
    // faster of the two past 2048 assignments
    const int64_t amax = E <= kPermFoldExperts ? kPermSmallFoldMax : (int64_t)16 * 64 * kPermSmallChunksPerWave;
    return A > 0 && A <= amax && (A + 63) / 64 * E <= kPermSmallCounts;
}

void launch_perm_index_small(const int32_t* topk_idx, int64_t A, int E, int k, int capacity, int32_t* offsets,
                             int32_t* inv_pos, int32_t* sorted_token, hipStream_t s) {
    int nbits = 0;
    while ((1 << nbits) <= E) ++nbits;  // ids 0..E (E = padding sentinel) fit in nbits bits
    int Ep = 1;
    while (Ep < E) Ep <<= 1;  // E <= 1024
    const size_t lds = (size_t)((A + 63) / 64) * E * sizeof(int);
    perm_index_small_kernel<<<1, 1024, lds, s>>>(topk_idx, A, E, k, nbits, Ep, capacity, offsets, inv_pos,
                                                 sorted_token);
}

void launch_perm_scan(const int32_t* tile_counts, int ntiles, int64_t A, int E, int capacity, int32_t* tile_base,
                      int32_t* offsets, hipStream_t s) {
    (void)A;
    int Ep = 1;
    while (Ep < E) Ep <<= 1;  // E <= 1024
    perm_scan_kernel<<<1, 1024, 0, s>>>(tile_counts, ntiles, E, Ep, capacity, tile_base, offsets);
}

void launch_perm_scatter(const void* x, const int32_t* inv_pos, int64_t T, int d, int k, int elem_bytes,
                         void* x_perm, hipStream_t s) {
    const unsigned nblk = (unsigned)((T + 3) / 4);
    perm_scatter_kernel<<<nblk, 256, 0, s>>>(static_cast<const uint8_t*>(x), inv_pos, T, d * elem_bytes, k,
                                             static_cast<uint8_t*>(x_perm));
}

void launch_perm_local(const int32_t* topk_idx, int64_t A, int E, int32_t* tile_counts, int32_t* local_rank,
                       hipStream_t s) {
    const unsigned ntiles = (unsigned)((A + kPermTile - 1) / kPermTile);
    int nbits = 0;
    while ((1 << nbits) <= E) ++nbits;  // ids 0..E (E = padding sentinel) fit in nbits bits
    const size_t lds = (size_t)(kPermTile / 64) * E * sizeof(int);
    perm_local_kernel<<<ntiles, 256, lds, s>>>(topk_idx, A, E, nbits, tile_counts, local_rank);
}

bool perm_fold_ok(int64_t A, int E, int k) {
    return E <= kPermFoldExperts && (A + kPermTile - 1) / kPermTile <= kPermFoldTiles && 4 * k <= kPermTile;
}

void launch_perm_place_scatter(const void* x, const int32_t* topk_idx, const int32_t* tile_counts,
                               const int32_t* tile_base, int32_t* offsets, int E, int capacity, int64_t T, int d,
                               int k, int elem_bytes, int32_t* inv_pos, int32_t* sorted_token, void* x_perm,
                               hipStream_t s) {
    const unsigned nblk = (unsigned)((T + 3) / 4);
    const int ntiles = (int)((T * k + kPermTile - 1) / kPermTile);
    const auto xb = static_cast<const uint8_t*>(x);
    const auto xp = static_cast<uint8_t*>(x_perm);
    if (x_perm == nullptr) {  // positions only
        const int64_t A = T * k;
        const unsigned nb = (unsigned)((A + 255) / 256);
        if (tile_base == nullptr)
            perm_place_kernel<true><<<nb, 256, 0, s>>>(topk_idx, tile_counts, nullptr, offsets, ntiles, E, capacity, A,
                                                       k, inv_pos, sorted_token);
        else
            perm_place_kernel<false><<<nb, 256, 0, s>>>(topk_idx, nullptr, tile_base, offsets, ntiles, E, capacity, A,
                                                        k, inv_pos, sorted_token);
        return;
    }
    if (tile_base == nullptr)
        perm_place_scatter_kernel<true><<<nblk, 256, 0, s>>>(xb, topk_idx, tile_counts, nullptr, offsets, ntiles, E,
                                                             capacity, T, d * elem_bytes, k, inv_pos, sorted_token, xp);
    else
        perm_place_scatter_kernel<false><<<nblk, 256, 0, s>>>(xb, topk_idx, nullptr, tile_base, offsets, ntiles, E,
                                                              capacity, T, d * elem_bytes, k, inv_pos, sorted_token,
                                                              xp);
}

}  // namespace moe
