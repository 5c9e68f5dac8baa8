// Two-stage top-k over float32 logits, with the soft-cap applied to the
// selected values ["Gemma 4 M4 Max kernel roadmap", K1: logit soft-capping;
// K2 step 6: on-GPU top-k reduction; "Metal kernel capability table",
// section 6: f32_topk_partial, a partial pass then a fan-in].
//
// Order: larger value first, equal values -> lower index first, NaN after
// every number.  Each (value, index) pair is packed into one 64-bit key whose
// unsigned order is exactly that order:
//   high 32 bits: the float's bits mapped to an increasing unsigned code
//                 (NaN -> 0, -0 -> +0), low 32 bits: 0xFFFFFFFF - index.
// A real key is never 0 (index < 2^31), so 0 means "nothing".  Keys are
// unique, so round r of a selection is "the largest key below the key chosen
// in round r-1": no per-element bookkeeping is needed.
//
// Stage 1: every wave owns a chunk of 64 KPL entries (KPL keys per lane, in
//          registers) and emits its k best, largest first.  For k <= 16 a
//          round is a lane-local masked maximum (a tree over KPL keys) plus
//          a DPP wave maximum, k rounds in all.  For larger k (with 4 keys
//          per lane, rows up to 262,144 entries) the wave sorts its 256 keys
//          with a bitonic network, at a cost that does not grow with k
//          (cross-lane steps are DPP moves and gfx950's permlane swaps).
//          KPL grows with N so that there are at most 1024 chunks.
// Stage 2: one 1024-thread workgroup per activation row.
//   k <= 16: a tournament over the sorted chunk lists in two levels: thread
//          t holds the head of list t (and the next few entries in
//          registers); each wave takes the k best of its 64 lists (a wave
//          maximum per round, the lane that owned it moves to its next
//          entry: keys are unique, so exactly one lane wins a round), then
//          wave 0 takes the k best of the 16 wave lists the same way.
//   k > 16: the list heads (each list's largest key) are sorted; T = the
//          k-th largest head.  At least k keys (those heads) are >= T, so
//          the k-th largest key overall is >= T and only keys >= T can win;
//          they lie in the k lists whose heads are >= T, at most k^2 keys
//          (about k for logits).  Those candidates are sorted and the first
//          k written.
// Very long rows (more than 4M entries, so more than 1024 chunks of 4096)
// fall back to a merge that rescans candidates from memory every round.
#include <stdint.h>

#include <mutex>

#include "qmv_device.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int kMergeThreads = 1024;
constexpr int kMergeWaves = kMergeThreads / kWave;
constexpr int kMaxLists = kMergeThreads;  // chunk lists the tournament takes
constexpr int kMaxCand = 64 * 64;         // candidates of stage 2: at most k^2, k <= 64
constexpr int kListRegs = 8;              // entries of its list a tournament thread keeps in registers
// Up to this k the selection runs k rounds (a wave maximum each); above it
// the chunks are sorted and stage 2 selects by threshold, whose cost does
// not grow with k.  Measured at 262,144 logits: k = 10 takes 13.0 us with
// rounds and 15.9 us sorted, k = 40 takes 35 us with rounds and 17 us
// sorted.
constexpr int kRoundsMaxK = 16;

// Branch-free (selects only), so that a run of keys can be formed after one
// batch of loads.
__device__ __forceinline__ uint64_t order_key(float v, uint32_t idx) {
    const uint32_t b = (v == 0.0f) ? 0u : __float_as_uint(v);  // -0 ranks with +0
    uint32_t code = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    code = (v != v) ? 0u : code;                                // NaN after every number
    return (static_cast<uint64_t>(code) << 32) | static_cast<uint64_t>(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Lanes the DPP pattern does not write keep 0, the identity of the max.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROW_MASK, 0xF, false));
}

// Maximum of an unsigned 32-bit value over the 64 lanes, returned to every
// lane.  Inclusive prefix maxima within each row of 16 lanes (row_shr 1, 2,
// 4, 8), then row 0's maximum into row 1 and row 2's into row 3 (row_bcast
// 15), then row 1's into rows 2-3 (row_bcast 31): lane 63 ends with the
// maximum of all lanes.
__device__ __forceinline__ uint32_t wave_max32(uint32_t v) {
    v = max(v, dpp32<0x111, 0xF>(v));
    v = max(v, dpp32<0x112, 0xF>(v));
    v = max(v, dpp32<0x114, 0xF>(v));
    v = max(v, dpp32<0x118, 0xF>(v));
    v = max(v, dpp32<0x142, 0xA>(v));
    v = max(v, dpp32<0x143, 0xC>(v));
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// Maximum of a 64-bit key over the wave: the largest high word first, then
// the largest low word among the lanes that hold it (two 32-bit reductions
// are shorter dependent chains than one on 64-bit values).  When a single
// lane holds the largest high word (equal values are rare), its low word is
// read directly and the second reduction is skipped.
__device__ __forceinline__ uint64_t wave_max64(uint64_t v) {
    const uint32_t hi = wave_max32(static_cast<uint32_t>(v >> 32));
    const uint64_t holders = __ballot(static_cast<uint32_t>(v >> 32) == hi);
    uint32_t lo;
    if (__popcll(holders) == 1) {
        lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)),
                                                             __ffsll(static_cast<unsigned long long>(holders)) - 1));
    } else {
        lo = wave_max32(static_cast<uint32_t>(v >> 32) == hi ? static_cast<uint32_t>(v) : 0u);
    }
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }

// v of lane ^ d, for d = 1, 2, 4, 8, 16, 32 (a constant once the sorting
// loops are unrolled), without the LDS crossbar: DPP quad permutes for 1 and
// 2, two row shifts for 4, a row rotation for 8, and gfx950's row and
// half-wave swaps for 16 and 32.
__device__ __forceinline__ uint32_t xor_lanes(uint32_t v, int d) {
    const int lane = threadIdx.x & (kWave - 1);
    switch (d) {
    case 1: return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, false));
    case 2: return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, false));
    case 4: {
        const uint32_t up = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x104, 0xF, 0xF, false));
        const uint32_t dn = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x114, 0xF, 0xF, false));
        return (lane & 4) ? dn : up;
    }
    case 8: return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x128, 0xF, 0xF, false));
    case 16: {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return ((lane >> 4) & 1) ? r[0] : r[1];
    }
    default: {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane >= 32) ? r[0] : r[1];
    }
    }
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int d) {
    const uint32_t lo = xor_lanes(static_cast<uint32_t>(v), d);
    const uint32_t hi = xor_lanes(static_cast<uint32_t>(v >> 32), d);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// One compare-exchange of a bitonic network, seen from one element: e is the
// element's index, d its partner's distance, s the size of the sequences
// being merged.  Sequences whose index has bit s clear are sorted largest
// first, so the final pass (s = n) leaves everything largest first.
__device__ __forceinline__ uint64_t bitonic_keep(uint64_t mine, uint64_t other, int e, int d, int s) {
    const bool lower = (e & d) == 0;
    const bool desc = (e & s) == 0;
    return (lower == desc) ? umax64(mine, other) : umin64(mine, other);
}

// Sorts the 64 NK keys of a wave, largest first: key[j] of lane l is element
// j * 64 + l.  Steps with distance >= 64 stay in the lane's registers, the
// others exchange with lane ^ d.
template <int NK>
__device__ __forceinline__ void wave_sort_desc(uint64_t (&key)[NK]) {
    const int lane = threadIdx.x & (kWave - 1);
    constexpr int n = kWave * NK;
#pragma unroll
    for (int s = 2; s <= n; s <<= 1) {
#pragma unroll
        for (int d = s >> 1; d > 0; d >>= 1) {
            if (d >= kWave) {
                const int dj = d / kWave;
#pragma unroll
                for (int j = 0; j < NK; ++j) {
                    if ((j ^ dj) > j) {
                        const uint64_t a = key[j], b = key[j ^ dj];
                        key[j] = bitonic_keep(a, b, j * kWave, d, s);
                        key[j ^ dj] = bitonic_keep(b, a, (j ^ dj) * kWave, d, s);
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < NK; ++j) key[j] = bitonic_keep(key[j], shfl_xor64(key[j], d), j * kWave + lane, d, s);
            }
        }
    }
}

// Sorts NB * 1024 keys held by a 1024-thread workgroup, largest first:
// key[j] of thread t is element j * 1024 + t.  Steps with distance < 64 are
// shuffles inside a wave, steps with distance >= 1024 stay in registers, the
// rest exchange through LDS (two buffers alternate, so one barrier a step).
template <int NB>
__device__ __forceinline__ void block_sort_desc(uint64_t (&key)[NB], uint64_t* lds /* 2 * NB * 1024 */) {
    constexpr int T = kMergeThreads;
    constexpr int n = T * NB;
    const int t = threadIdx.x;
    int buf = 0;
#pragma unroll
    for (int s = 2; s <= n; s <<= 1) {
#pragma unroll
        for (int d = s >> 1; d > 0; d >>= 1) {
            if (d >= T) {
                const int dj = d / T;
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    if ((j ^ dj) > j) {
                        const uint64_t a = key[j], b = key[j ^ dj];
                        key[j] = bitonic_keep(a, b, j * T, d, s);
                        key[j ^ dj] = bitonic_keep(b, a, (j ^ dj) * T, d, s);
                    }
                }
            } else if (d >= kWave) {
                uint64_t* B = lds + buf * (NB * T);
#pragma unroll
                for (int j = 0; j < NB; ++j) B[j * T + t] = key[j];
                __syncthreads();
#pragma unroll
                for (int j = 0; j < NB; ++j) key[j] = bitonic_keep(key[j], B[j * T + (t ^ d)], j * T + t, d, s);
                buf ^= 1;
            } else {
#pragma unroll
                for (int j = 0; j < NB; ++j) key[j] = bitonic_keep(key[j], shfl_xor64(key[j], d), j * T + t, d, s);
            }
        }
    }
}

// Largest of the NK keys below `bound` (0 if none), as a balanced tree.
template <int NK>
__device__ __forceinline__ uint64_t masked_max(const uint64_t (&key)[NK], uint64_t bound) {
    uint64_t t[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) t[i] = key[i] < bound ? key[i] : 0ull;
#pragma unroll
    for (int w = 1; w < NK; w *= 2)
#pragma unroll
        for (int i = 0; i + w < NK; i += 2 * w) t[i] = umax64(t[i], t[i + w]);
    return t[0];
}

// k rounds over NK keys per lane held in registers; lane r writes the
// round-r winner to out[r] (r < k): the k largest keys, largest first.
template <int NK>
__device__ __forceinline__ void wave_select(const uint64_t (&key)[NK], int k, uint64_t* out) {
    const int lane = threadIdx.x & (kWave - 1);
    uint64_t bound = ~0ull;
    for (int r = 0; r < k; ++r) {
        const uint64_t best = wave_max64(masked_max(key, bound));
        if (lane == r) out[r] = best;
        bound = best;
    }
}

template <int KPL>
__global__ __launch_bounds__(kBlockThreads)
void topk_chunk_kernel(const float* __restrict__ y, int64_t N, int k, int nwchunks,
                       uint64_t* __restrict__ cand) {
    const int m = blockIdx.y;
    const int c = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;  // this wave's chunk
    if (c >= nwchunks) return;                                        // whole wave leaves together
    const int lane = threadIdx.x & (kWave - 1);
    const float* ym = y + static_cast<int64_t>(m) * N;
    // all KPL loads first (indices past N read the last entry again), then
    // the keys: one memory round trip instead of one per key
    float v[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int64_t idx = (static_cast<int64_t>(c) * KPL + i) * kWave + lane;
        v[i] = ym[idx < N ? idx : N - 1];
    }
    uint64_t key[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int64_t idx = (static_cast<int64_t>(c) * KPL + i) * kWave + lane;
        key[i] = idx < N ? order_key(v[i], static_cast<uint32_t>(idx)) : 0ull;
    }
    uint64_t* out = cand + (static_cast<int64_t>(m) * nwchunks + c) * k;
    if (KPL == 4 && k > kRoundsMaxK) {
        wave_sort_desc(key);
        if (lane < k) out[lane] = key[0];  // elements 0 .. k-1 of the sorted chunk
    } else {
        wave_select(key, k, out);
    }
}

// The top-p draw of one row by one whole wave, lane i holding the i-th
// largest capped value z and its index (lanes >= k: have = false)
// ["Gemma 4 M4 Max kernel roadmap", K5: top-k40 / top-p token selection on
// the device after the tied projection]:
//   w_i = exp((z_i - z_0) / T) for i < k (z sorted, largest first; NaN -> 0),
//   n   = the smallest count whose prefix sum reaches top_p * sum(w)  (n >= 1),
//   j   = the first i < n whose prefix sum exceeds u * (prefix sum of n),
//   token = index_j.
// The prefix sums are one inclusive wave scan (a fixed order, so the draw is
// reproducible).
__device__ void draw_topp(float z, int32_t idx, bool have, int64_t m, int k, const TopPDraw& D) {
    const int lane = threadIdx.x & (kWave - 1);
    const float z0 = __shfl(z, 0, kWave);
    float w = 0.0f;
    if (have && z == z && z0 == z0) w = expf((z - z0) / D.temperature);
    float cum = w;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const float t = __shfl_up(cum, o, kWave);
        if (lane >= o) cum += t;
    }
    const float total = __shfl(cum, kWave - 1, kWave);
    int n = 1, j = 0;
    if (total > 0.0f) {
        const uint64_t reach = __ballot(have && cum >= D.top_p * total);
        n = reach ? __ffsll(static_cast<unsigned long long>(reach)) : k;  // first lane reaching, plus one
        const float cut = __shfl(cum, n - 1, kWave);
        const float target = D.u[m] * cut;
        const uint64_t past = __ballot(lane < n && cum > target);
        j = past ? __ffsll(static_cast<unsigned long long>(past)) - 1 : n - 1;
    }
    const int32_t tok = __shfl(idx, j, kWave);
    if (lane == 0) {
        D.token[m] = tok;
        D.nucleus[m] = n;
    }
}

// Tournament over nlists <= 1024 sorted lists of k keys.
__global__ __launch_bounds__(kMergeThreads)
void topk_tournament_kernel(const float* __restrict__ y, int64_t N, int k, int nlists, float softcap,
                            const uint64_t* __restrict__ cand, float* __restrict__ top_val,
                            int32_t* __restrict__ top_idx, TopPDraw draw) {
    // Level 1: every wave runs its own tournament over its 64 lists (a wave
    // maximum per round, no workgroup barrier) and keeps its k winners in
    // LDS.  Level 2: wave 0 runs the tournament over the 16 waves' lists.
    __shared__ uint64_t wlist[kMergeWaves][64];
    const int m = blockIdx.x;
    const int t = threadIdx.x;
    const int w = t / kWave;
    const int lane = t & (kWave - 1);
    const uint64_t* list = cand + (static_cast<int64_t>(m) * nlists + t) * k;
    const bool mine = t < nlists;
    uint64_t buf[kListRegs];
#pragma unroll
    for (int i = 0; i < kListRegs; ++i) buf[i] = (mine && i < k) ? list[i] : 0ull;
    int next = kListRegs;  // next entry of the list to fetch
    for (int r = 0; r < k; ++r) {
        const uint64_t g = wave_max64(buf[0]);
        if (lane == 0) wlist[w][r] = g;
        if (buf[0] == g && g != 0ull) {  // keys are unique: one lane
#pragma unroll
            for (int i = 0; i + 1 < kListRegs; ++i) buf[i] = buf[i + 1];
            buf[kListRegs - 1] = 0ull;
            // Refill only when the register copy runs dry: a load issued every
            // round would make the next round wait for it (the wait counts
            // are per wave), and a list rarely gives more than a few winners.
            if (buf[0] == 0ull && next < k) {
#pragma unroll
                for (int i = 0; i < kListRegs; ++i) buf[i] = (next + i < k) ? list[next + i] : 0ull;
                next += kListRegs;
            }
        }
    }
    __syncthreads();
    if (w != 0) return;
    int pos = 0;  // lane l < 16 reads wave l's list
    uint64_t head = lane < kMergeWaves ? wlist[lane][0] : 0ull;
    uint64_t mine_key = 0ull;  // lane r keeps the winner of round r
    for (int r = 0; r < k; ++r) {
        const uint64_t g = wave_max64(head);
        if (lane == r) mine_key = g;
        if (head == g && g != 0ull) {
            ++pos;
            head = pos < k ? wlist[lane][pos] : 0ull;
        }
    }
    float z = 0.0f;
    int32_t zi = -1;
    if (lane < k) {
        // k <= N guarantees a real key every round; a zero key would mean
        // "nothing left" and is never dereferenced.
        const uint64_t g = mine_key;
        const uint32_t idx = 0xFFFFFFFFu - static_cast<uint32_t>(g);
        const bool real = g != 0ull && idx < static_cast<uint64_t>(N);
        const float v = real ? y[static_cast<int64_t>(m) * N + idx] : __builtin_nanf("");
        zi = real ? static_cast<int32_t>(idx) : -1;
        z = softcap * tanhf(v / softcap);
        top_idx[static_cast<int64_t>(m) * k + lane] = zi;
        top_val[static_cast<int64_t>(m) * k + lane] = z;
    }
    if (draw.token) draw_topp(z, zi, lane < k, m, k, draw);
}

// Stage 2 over nlists <= 1024 sorted lists of k keys (chunk: entries per
// list's chunk, to find a key's list from its index).
__global__ __launch_bounds__(kMergeThreads)
void topk_select_kernel(const float* __restrict__ y, int64_t N, int k, int nlists, int chunk, float softcap,
                        const uint64_t* __restrict__ cand, float* __restrict__ top_val,
                        int32_t* __restrict__ top_idx, TopPDraw draw) {
    __shared__ uint64_t lds[2 * kMaxCand];  // sort buffers, then the candidates
    __shared__ uint64_t sh_T;
    __shared__ int sh_off[kWave + 1];
    const int m = blockIdx.x;
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const uint64_t* cm = cand + static_cast<int64_t>(m) * nlists * k;

    // 1. sort the heads; T = the k-th largest (0 if fewer than k lists)
    uint64_t h[1] = {t < nlists ? cm[static_cast<int64_t>(t) * k] : 0ull};
    block_sort_desc<1>(h, lds);
    if (t == k - 1) sh_T = h[0];
    __syncthreads();
    const uint64_t T = sh_T;

    // 2. thread t < k holds the t-th largest head; its list gives the keys
    //    >= T, a prefix (lists are sorted).  The k lists are copied into LDS
    //    with one round of loads, counted there, and their keys >= T packed
    //    into the candidate buffer.
    __shared__ int sh_list[kWave];
    uint64_t* lists = lds;             // [k][k]
    uint64_t* cbuf = lds + kMaxCand;   // [C]
    if (t < k) {
        sh_list[t] = h[0] != 0ull ? static_cast<int>((0xFFFFFFFFu - static_cast<uint32_t>(h[0])) /
                                                     static_cast<uint32_t>(chunk))
                                  : -1;
    }
    __syncthreads();
    for (int e = t; e < k * k; e += kMergeThreads) {
        const int o = e / k;
        const int l = sh_list[o];
        lists[e] = l >= 0 ? cm[static_cast<int64_t>(l) * k + (e - o * k)] : 0ull;
    }
    __syncthreads();
    int cnt = 0;
    if (t < k) {
        for (int i = 0; i < k; ++i) {
            const uint64_t v = lists[t * k + i];
            cnt += (v >= T && v != 0ull) ? 1 : 0;
        }
    }
    if (t < kWave) {
        // exclusive prefix of the counts over wave 0 (k <= 64 lanes)
        int inc = cnt;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int v = __shfl_up(inc, o, kWave);
            if (lane >= o) inc += v;
        }
        sh_off[lane + 1] = inc;
        if (lane == 0) sh_off[0] = 0;
    }
    __syncthreads();
    const int C = sh_off[kWave];  // <= k^2 <= kMaxCand
    if (t < k) {
        const int off = sh_off[t];
        for (int i = 0; i < cnt; ++i) cbuf[off + i] = lists[t * k + i];
    }
    __syncthreads();

    // 3. sort the C candidates; the first k are the result
    uint64_t best = 0ull;  // thread r < k: the r-th largest key
    if (C <= kWave) {
        if (t < kWave) {
            uint64_t key[1] = {lane < C ? cbuf[lane] : 0ull};
            wave_sort_desc(key);
            best = key[0];
        }
    } else if (C <= 4 * kWave) {
        if (t < kWave) {
            uint64_t key[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) key[j] = (j * kWave + lane < C) ? cbuf[j * kWave + lane] : 0ull;
            wave_sort_desc(key);
            best = key[0];
        }
    } else {
        uint64_t key[kMaxCand / kMergeThreads];
#pragma unroll
        for (int j = 0; j < kMaxCand / kMergeThreads; ++j)
            key[j] = (j * kMergeThreads + t < C) ? cbuf[j * kMergeThreads + t] : 0ull;
        __syncthreads();  // the candidates are in registers: the buffers are free
        block_sort_desc(key, lds);
        best = key[0];
    }
    if (t < kWave) {  // wave 0; k <= 64
        float z = 0.0f;
        int32_t zi = -1;
        if (t < k) {
            // k <= N guarantees a real key at every rank < k; a zero key would
            // mean "nothing left" and is never dereferenced.
            const uint32_t idx = 0xFFFFFFFFu - static_cast<uint32_t>(best);
            const bool real = best != 0ull && idx < static_cast<uint64_t>(N);
            const float v = real ? y[static_cast<int64_t>(m) * N + idx] : __builtin_nanf("");
            zi = real ? static_cast<int32_t>(idx) : -1;
            z = softcap * tanhf(v / softcap);
            top_idx[static_cast<int64_t>(m) * k + t] = zi;
            top_val[static_cast<int64_t>(m) * k + t] = z;
        }
        if (draw.token) draw_topp(z, zi, t < k, m, k, draw);
    }
}

// More than 1024 lists: every wave scans its share of the candidates from
// memory each round; wave 0 then selects among the waves' winners.
__global__ __launch_bounds__(kMergeThreads)
void topk_merge_scan_kernel(const float* __restrict__ y, int64_t N, int k, int nlists, float softcap,
                            const uint64_t* __restrict__ cand, float* __restrict__ top_val,
                            int32_t* __restrict__ top_idx) {
    __shared__ uint64_t stage[kMergeWaves * 64];
    const int m = blockIdx.x;
    const int w = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t ncand = static_cast<int64_t>(nlists) * k;
    const uint64_t* cm = cand + static_cast<int64_t>(m) * ncand;
    const int64_t per = (ncand + kMergeWaves - 1) / kMergeWaves;
    const int64_t lo = w * per;
    const int64_t hi = (lo + per < ncand) ? lo + per : ncand;
    uint64_t bound = ~0ull;
    for (int r = 0; r < k; ++r) {
        uint64_t best = 0ull;
        for (int64_t j = lo + lane; j < hi; j += kWave) {
            const uint64_t v = cm[j];
            if (v < bound) best = umax64(best, v);
        }
        best = wave_max64(best);
        if (lane == r) stage[w * 64 + r] = best;
        bound = best;
    }
    __syncthreads();
    if (w == 0) {
        uint64_t key[kMergeWaves];
#pragma unroll
        for (int i = 0; i < kMergeWaves; ++i) key[i] = lane < k ? stage[i * 64 + lane] : 0ull;
        uint64_t b2 = ~0ull;
        for (int r = 0; r < k; ++r) {
            const uint64_t best = wave_max64(masked_max(key, b2));
            if (lane == 0) {
                const uint32_t idx = 0xFFFFFFFFu - static_cast<uint32_t>(best);
                const bool real = best != 0ull && idx < static_cast<uint64_t>(N);
                const float v = real ? y[static_cast<int64_t>(m) * N + idx] : __builtin_nanf("");
                top_idx[static_cast<int64_t>(m) * k + r] = real ? static_cast<int32_t>(idx) : -1;
                top_val[static_cast<int64_t>(m) * k + r] = softcap * tanhf(v / softcap);
            }
            b2 = best;
        }
    }
}

// Keys per lane of stage 1: the smallest of 4, 16, 64 that leaves at most
// 1024 chunks (64 for longer rows).
int keys_per_lane(int64_t N) {
    if (N <= int64_t{kMaxLists} * kWave * 4) return 4;
    if (N <= int64_t{kMaxLists} * kWave * 16) return 16;
    return 64;
}

int64_t wave_chunks_of(int64_t N) {
    const int64_t chunk = static_cast<int64_t>(kWave) * keys_per_lane(N);
    return (N + chunk - 1) / chunk;
}

size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

// ---------------------------------------------------------- sampling
// The draw of draw_topp from k given pairs per row (one wave per row): the
// path of logits_sample when the selection kernel cannot make it, and the
// test export.
__global__ __launch_bounds__(kWave)
void sample_topp_kernel(const float* __restrict__ top_val, const int32_t* __restrict__ top_idx, int k,
                        TopPDraw draw) {
    const int64_t m = blockIdx.x;
    const int lane = threadIdx.x;
    const bool have = lane < k;
    const float z = have ? top_val[m * k + lane] : 0.0f;
    const int32_t zi = have ? top_idx[m * k + lane] : -1;
    draw_topp(z, zi, have, m, k, draw);
}

}  // namespace

size_t topk_ws_bytes(int64_t N, int64_t M, int k) {
    const size_t ybytes = align256(static_cast<size_t>(N) * static_cast<size_t>(M) * sizeof(float));
    const size_t cbytes =
        static_cast<size_t>(M) * static_cast<size_t>(wave_chunks_of(N)) * static_cast<size_t>(k) * sizeof(uint64_t);
    return ybytes + align256(cbytes);
}

hipError_t launch_topk(const float* y, float* top_val, int32_t* top_idx, int64_t N, int64_t M, int k,
                       float softcap, void* ws, hipStream_t stream, const TopPDraw& draw, bool* drawn) {
    if (drawn) *drawn = false;
    const int nwchunks = static_cast<int>(wave_chunks_of(N));
    uint64_t* cand = reinterpret_cast<uint64_t*>(
        static_cast<char*>(ws) + align256(static_cast<size_t>(N) * static_cast<size_t>(M) * sizeof(float)));
    const unsigned blocks = static_cast<unsigned>((nwchunks + kWavesPerBlock - 1) / kWavesPerBlock);
    const dim3 grid(blocks, static_cast<unsigned>(M));
    switch (keys_per_lane(N)) {
    case 4:
        hipLaunchKernelGGL(topk_chunk_kernel<4>, grid, dim3(kBlockThreads), 0, stream, y, N, k, nwchunks, cand);
        break;
    case 16:
        hipLaunchKernelGGL(topk_chunk_kernel<16>, grid, dim3(kBlockThreads), 0, stream, y, N, k, nwchunks, cand);
        break;
    default:
        hipLaunchKernelGGL(topk_chunk_kernel<64>, grid, dim3(kBlockThreads), 0, stream, y, N, k, nwchunks, cand);
        break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (nwchunks <= kMaxLists && k > kRoundsMaxK) {
        hipLaunchKernelGGL(topk_select_kernel, dim3(static_cast<unsigned>(M)), dim3(kMergeThreads), 0, stream,
                           y, N, k, nwchunks, kWave * keys_per_lane(N), softcap, cand, top_val, top_idx, draw);
        if (drawn) *drawn = draw.token != nullptr;
    } else if (nwchunks <= kMaxLists) {
        hipLaunchKernelGGL(topk_tournament_kernel, dim3(static_cast<unsigned>(M)), dim3(kMergeThreads), 0, stream,
                           y, N, k, nwchunks, softcap, cand, top_val, top_idx, draw);
        if (drawn) *drawn = draw.token != nullptr;
    } else {
        hipLaunchKernelGGL(topk_merge_scan_kernel, dim3(static_cast<unsigned>(M)), dim3(kMergeThreads), 0, stream,
                           y, N, k, nwchunks, softcap, cand, top_val, top_idx);
    }
    return hipGetLastError();
}

// Workspace of logits_topk_noalloc, for callers that cannot allocate: a
// file-scope device array of kStaticScratchBytes, one copy per GPU (each
// device that loads the library holds its own until the process ends).  Host
// code never uses the array's name as an address: that is a host-side
// stand-in.  static_scratch() asks the runtime for the device address of the
// current device's copy once per device and hands that out.
namespace {
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
}  // namespace

void* static_scratch() {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* ptr[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        ptr[dev] = p;
    }
    return ptr[dev];
}

hipError_t launch_sample(const float* top_val, const int32_t* top_idx, const float* u, int32_t* token,
                         int32_t* nucleus, int64_t M, int k, float temperature, float top_p, hipStream_t stream) {
    TopPDraw draw;
    draw.u = u;
    draw.token = token;
    draw.nucleus = nucleus;
    draw.temperature = temperature;
    draw.top_p = top_p;
    hipLaunchKernelGGL(sample_topp_kernel, dim3(static_cast<unsigned>(M)), dim3(kWave), 0, stream, top_val, top_idx, k,
                       draw);
    return hipGetLastError();
}

}  // namespace qmv
