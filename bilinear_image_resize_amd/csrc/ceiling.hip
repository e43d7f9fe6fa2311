// Launch and bandwidth ceilings of one MI355X, measured beside the library.
//
// A measurement program, not part of the library's interface: it times the
// library's own entry points (resize_linear, resize_copy_bytes) through the
// C ABI - including the 4K RGB frame on 1 to 4 streams and the exact 2:1
// kernel over a range of frame heights - plus a few kernels of its own that bound what any kernel of the
// same shape can reach (an empty grid, a read-only stream, a stand-in
// with the exact 2:1 kernel's loads, stores and grid that records when each
// workgroup starts and ends, stand-ins with the exact 2x kernel's grid
// and byte mix, and one with the float RGBA enlargement's byte mix).  It
// prints one JSON object per line.
//
// Timing follows the method of "From Prototype to Performance: Optimizing
// OpenCV Resize on Volcanic GPUs" (section "Measure performance carefully":
// device events, useful bytes = input + output), with two additions: every
// timed run rotates over enough buffers to defeat the 256 MB Infinity Cache,
// and a bounded spin kernel holds the stream until all launches of the run
// are enqueued, so the events time launches that follow each other back to
// back rather than the host's enqueue rate.
//
//     mi_resize_ceiling [section ...]    (all sections by default)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "mi_resize.h"

#define CK(x)                                                                                  \
    do {                                                                                       \
        hipError_t e_ = (x);                                                                   \
        if (e_ != hipSuccess) {                                                                \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);      \
            exit(1);                                                                           \
        }                                                                                      \
    } while (0)

namespace {

constexpr double kPeakGBps = 8000.0;          // MI355X HBM3E, published
constexpr size_t kRotateBytes = 600u << 20;   // > 2 x the 256 MB Infinity Cache

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ void empty_kernel() {}

// Spins for `ticks` of the constant-rate wall clock (100 MHz), then exits.
__global__ void hold_kernel(unsigned long long ticks)
{
    const unsigned long long t0 = wall_clock64();
    while (wall_clock64() - t0 < ticks) __builtin_amdgcn_s_sleep(8);
}

// Reads n16 16-byte units with non-temporal loads; stores only if the xor of
// everything equals a constant it practically never equals (the loads
// cannot be dropped), and then inside dst's first dn16 units.
__global__ __launch_bounds__(256) void read_only(const u32x4 *__restrict__ s, u32x4 *__restrict__ d,
                                                 long long n16, long long dn16)
{
    const long long stride = (long long)gridDim.x * 256;
    u32x4 acc = {0, 0, 0, 0};
    long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride)
        acc ^= __builtin_nontemporal_load(s + i) ^ __builtin_nontemporal_load(s + i + stride) ^
               __builtin_nontemporal_load(s + i + 2 * stride) ^
               __builtin_nontemporal_load(s + i + 3 * stride);
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(s + i);
    if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u && acc.z == 0x2545f491u)
        d[((long long)blockIdx.x * 256 + threadIdx.x) % dn16] = acc;
}

// Stand-in for the exact 2:1 RGB kernel on a 2160 x 3840 frame: the same
// 1-D grid of two-wave workgroups over (row, segment) items, each wave
// reading its segment of two source rows with 16-byte non-temporal loads
// and writing the rounded 2x2 means (bytewise here).  Lane 0 of each wave
// records its start and end on the wall clock.
constexpr int kTrH = 2160, kTrW = 3840, kTrDW = kTrW / 2, kTrSegs = 8;
constexpr int kTrSegPx = 256, kTrSB = 2 * kTrSegPx * 3;

__global__ __launch_bounds__(128) void traced_half_rgb(const uint8_t *__restrict__ src,
                                                       uint8_t *__restrict__ dst,
                                                       unsigned long long *__restrict__ tr)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds_all[2][2 * kTrSB];
    const unsigned long long t0 = wall_clock64();
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    uint8_t *lds = lds_all[wave];
    const unsigned item = blockIdx.x * 2 + wave;
    if (item >= (unsigned)kTrSegs * (kTrH / 2)) return;
    const int row = item / kTrSegs, seg = item % kTrSegs;
    const int seg_px = min(kTrSegPx, kTrDW - seg * kTrSegPx);
    const int n16 = seg_px * 6 / 16;
    const uint8_t *s0 = src + (size_t)(2 * row) * (kTrW * 3) + (size_t)seg * kTrSB;
    const uint8_t *s1 = s0 + kTrW * 3;
    u32x4 va[2], vb[2];
    for (int i = 0; i < 2; ++i) {
        const int k = lane + 64 * i;
        if (k < n16) {
            va[i] = __builtin_nontemporal_load((const u32x4 *)(s0 + 16 * k));
            vb[i] = __builtin_nontemporal_load((const u32x4 *)(s1 + 16 * k));
        }
    }
    for (int i = 0; i < 2; ++i) {
        const int k = lane + 64 * i;
        if (k < n16) {
            *(u32x4 *)(lds + 16 * k) = va[i];
            *(u32x4 *)(lds + kTrSB + 16 * k) = vb[i];
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane * 4 < seg_px) {
        const uint8_t *a = lds + 24 * lane, *b = lds + kTrSB + 24 * lane;
        uint8_t *o = dst + (size_t)row * (kTrDW * 3) + (size_t)seg * kTrSegPx * 3 + 12 * lane;
        for (int k = 0; k < 12; ++k) {
            const int p = 2 * k - k % 3;
            o[k] = (uint8_t)((a[p] + a[p + 3] + b[p] + b[p + 3] + 2) >> 2);
        }
    }
    if (lane == 0) {
        tr[2 * item] = t0;
        tr[2 * item + 1] = wall_clock64();
    }
}

// Stand-ins for the exact 2x one-channel kernel on a 1080 x 1920 frame
// (output 2160 x 3840) with its grid: four-wave workgroups over (512-pixel
// segment, group of four row gaps), renumbered so that each XCD takes a
// contiguous run, one wave per gap, each lane owning 8 source columns and so
// 16 output bytes of each of the gap's two output rows.  Gap g (-1 .. 1079)
// lies between source rows g and g + 1 and writes output rows 2g + 1 and
// 2g + 2 where they exist.  READ = false writes without reading anything;
// READ = true first loads, as the kernel does, a 16-byte window around the
// lane's 8 bytes of both source rows (clamped into the frame) and writes
// bytes made from them.  Together they bound what any kernel with this byte
// mix and grid can reach.
constexpr int kU2H = 1080, kU2W = 1920, kU2Segs = 4, kU2Gaps = kU2H + 1;
constexpr int kU2GapGroups = (kU2Gaps + 3) / 4;

__device__ __forceinline__ unsigned xcd_run(unsigned lin, unsigned nwg)
{
    const unsigned xcd = lin & 7;
    return xcd * (nwg >> 3) + min(xcd, nwg & 7) + (lin >> 3);
}

template <bool READ>
__global__ __launch_bounds__(256) void up2_standin(const uint8_t *__restrict__ src,
                                                   uint8_t *__restrict__ dst)
{
    const unsigned wid = xcd_run(blockIdx.x, gridDim.x);
    const int seg = (int)(wid % kU2Segs), grp = (int)(wid / kU2Segs);
    const int gap = grp * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) - 1;
    const int x0 = seg * 512 + 8 * ((int)threadIdx.x & 63);
    if (gap >= kU2H || x0 >= kU2W) return;
    u32x4 o = {(unsigned)gap, (unsigned)x0, 0x01010101u, 0x02020202u};
    if (READ) {
        const int ra = gap < 0 ? 0 : gap, rb = gap + 1 > kU2H - 1 ? kU2H - 1 : gap + 1;
        const int xw = x0 < 4 ? 0 : (x0 + 12 > kU2W ? kU2W - 16 : x0 - 4);
        u32x4 a, b;   // 4-byte aligned windows, as in the kernel
        __builtin_memcpy(&a, __builtin_assume_aligned(src + (size_t)ra * kU2W + xw, 4), 16);
        __builtin_memcpy(&b, __builtin_assume_aligned(src + (size_t)rb * kU2W + xw, 4), 16);
        o = a ^ b.yzwx;
    }
    if (2 * gap + 1 >= 0)
        __builtin_nontemporal_store(o, (u32x4 *)(dst + (size_t)(2 * gap + 1) * (2 * kU2W) + 2 * x0));
    if (2 * gap + 2 <= 2 * kU2H - 1)
        __builtin_nontemporal_store(o ^ 0x5a5a5a5au,
                                    (u32x4 *)(dst + (size_t)(2 * gap + 2) * (2 * kU2W) + 2 * x0));
}

int g_wall_khz = 100000;

void hold(hipStream_t st, int launches)
{
    // about 8 us per launch to come, enough for the host to enqueue them
    const unsigned long long ticks = (unsigned long long)g_wall_khz / 1000ull * 8ull * launches;
    hipLaunchKernelGGL(hold_kernel, dim3(1), dim3(64), 0, st, ticks);
}

// Median over 5 runs of the per-launch time (us) of `iters` launches that
// run back to back on S streams (launch i on stream i % S).
template <typename F>
double time_us(F launch, int iters, int S, hipStream_t *st)
{
    hipEvent_t a, b, ev[8];
    CK(hipEventCreate(&a));
    CK(hipEventCreate(&b));
    for (int s = 0; s < S; ++s) CK(hipEventCreate(&ev[s]));
    for (int i = 0; i < 2 * S + 8; ++i) launch(i, st[i % S]);
    CK(hipDeviceSynchronize());
    std::vector<double> r;
    for (int rep = 0; rep < 5; ++rep) {
        hold(st[0], iters);
        CK(hipEventRecord(a, st[0]));
        for (int s = 1; s < S; ++s) CK(hipStreamWaitEvent(st[s], a, 0));
        for (int i = 0; i < iters; ++i) launch(i, st[i % S]);
        for (int s = 1; s < S; ++s) {
            CK(hipEventRecord(ev[s], st[s]));
            CK(hipStreamWaitEvent(st[0], ev[s], 0));
        }
        CK(hipEventRecord(b, st[0]));
        CK(hipEventSynchronize(b));
        float ms;
        CK(hipEventElapsedTime(&ms, a, b));
        r.push_back(ms * 1e3 / iters);
    }
    CK(hipGetLastError());
    CK(hipEventDestroy(a));
    CK(hipEventDestroy(b));
    for (int s = 0; s < S; ++s) CK(hipEventDestroy(ev[s]));
    std::sort(r.begin(), r.end());
    return r[2];
}

// Pseudo-random bytes (an integer hash of the index): kernels that do much
// arithmetic per byte run measurably slower on random than on constant data
// (the thumbnail batch 47.8 vs 44.4 us), so no buffer here is left constant.
// Stand-in with the float RGBA enlargement's byte mix (4320 x 7680 -> 5927 x
// 3153, 16-byte pixels): workgroup w reads source units [256 L w, 256 L (w +
// 1)), L lane-strided 16-byte loads per lane, all in flight together, and
// writes output units [o(w), o(w + 1)), o(w) = w nd16 / groups, lane
// strided, with non-temporal stores of values that depend on every load of
// the lane.  Every source byte is read once and every output byte written
// once, in coalesced runs; ns16 is a multiple of 256 L (the caller checks).
template <int L>
__global__ __launch_bounds__(256) void mix_standin(const u32x4 *__restrict__ s, u32x4 *__restrict__ d,
                                                   long long nd16)
{
    const long long s0 = (long long)blockIdx.x * (256 * L);
    u32x4 acc = {0, 0, 0, 0};
    u32x4 v[L];
#pragma unroll
    for (int r = 0; r < L; ++r) v[r] = s[s0 + threadIdx.x + 256 * r];
#pragma unroll
    for (int r = 0; r < L; ++r) acc ^= v[r];
    const long long o0 = (long long)blockIdx.x * nd16 / gridDim.x;
    const long long o1 = ((long long)blockIdx.x + 1) * nd16 / gridDim.x;
    for (long long o = o0 + threadIdx.x; o < o1; o += 256) {
        acc.x += 1u;
        __builtin_nontemporal_store(acc, d + o);
    }
}

__global__ void fill_hash(uint32_t *p, size_t n, uint32_t seed)
{
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
        uint32_t x = (uint32_t)i * 0x9E3779B1u ^ seed;
        x ^= x >> 15;
        x *= 0x2C1B3C6Du;
        x ^= x >> 12;
        x *= 0x297A2D39u;
        x ^= x >> 15;
        p[i] = x;
    }
}

struct Ring {
    std::vector<uint8_t *> p;
    Ring(size_t bytes, int n)
    {
        for (int i = 0; i < n; ++i) {
            uint8_t *q;
            CK(hipMalloc(&q, bytes));
            CK(hipMemset(q, 0, bytes));
            hipLaunchKernelGGL(fill_hash, dim3(2048), dim3(256), 0, 0, (uint32_t *)q, bytes / 4,
                               0x5bd1e995u * (uint32_t)(i + 1));
            p.push_back(q);
        }
        CK(hipDeviceSynchronize());
    }
    ~Ring()
    {
        for (auto q : p) (void)hipFree(q);
    }
};

void copy_vs_size(hipStream_t *st)
{
    // bytes each way; 15552000 is half of the 4K RGB resize's 31,104,000
    for (long long n : {2ll << 20, 8ll << 20, 15552000ll, 32ll << 20, 128ll << 20, 415ll << 20}) {
        const int pairs = std::max<int>(2, (int)(kRotateBytes / (2 * n)) + 1);
        Ring ring((size_t)n, 2 * pairs);
        auto f = [&](int i, hipStream_t s) {
            const int j = i % pairs;
            if (resize_copy_bytes(ring.p[2 * j], ring.p[2 * j + 1], n, s) != 0) exit(2);
        };
        const int iters = n >= (128ll << 20) ? 40 : 400;
        const double us = time_us(f, iters, 1, st);
        printf("{\"section\": \"copy_vs_size\", \"bytes_each_way\": %lld, \"bytes_moved\": %lld, "
               "\"us\": %.3f, \"GBps\": %.1f, \"frac_of_peak\": %.4f}\n",
               n, 2 * n, us, 2.0 * n / (us * 1e3), 2.0 * n / (us * 1e3) / kPeakGBps);
    }
}

void empty_grids(hipStream_t *st)
{
    struct G { unsigned x, y, t; const char *what; };
    const G grids[] = {{8640, 1, 64, "8640 one-wave workgroups (1-D)"},
                       {8, 1080, 64, "8 x 1080 one-wave workgroups (2-D)"},
                       {4320, 1, 128, "4320 two-wave workgroups: the 4K RGB 2:1 grid"},
                       {2160, 1, 256, "2160 four-wave workgroups"},
                       {2048, 1, 256, "2048 four-wave workgroups"},
                       {256, 1, 256, "256 four-wave workgroups"},
                       {1, 1, 64, "one wave"}};
    for (const G &g : grids) {
        auto f = [&](int, hipStream_t s) {
            hipLaunchKernelGGL(empty_kernel, dim3(g.x, g.y), dim3(g.t), 0, s);
        };
        printf("{\"section\": \"empty_grid\", \"grid\": \"%s\", \"us\": %.3f}\n", g.what,
               time_us(f, 400, 1, st));
    }
}

void read_only_stream(hipStream_t *st)
{
    const long long n = 24883200;   // the 4K RGB frame's source bytes
    const int bufs = (int)(kRotateBytes / n) + 1;
    Ring ring((size_t)n, bufs);
    Ring sink(4096, 1);
    for (unsigned grid : {1024u, 2048u, 4096u}) {
        auto f = [&](int i, hipStream_t s) {
            hipLaunchKernelGGL(read_only, dim3(grid), dim3(256), 0, s,
                               (const u32x4 *)ring.p[i % bufs], (u32x4 *)sink.p[0], n / 16,
                               4096ll / 16);
        };
        const double us = time_us(f, 400, 1, st);
        printf("{\"section\": \"read_only\", \"bytes\": %lld, \"grid\": %u, \"us\": %.3f, "
               "\"GBps\": %.1f, \"frac_of_peak\": %.4f}\n",
               n, grid, us, n / (us * 1e3), n / (us * 1e3) / kPeakGBps);
    }
}

void resize_4k(hipStream_t *st)
{
    const long long sb = 24883200, db = 6220800;
    const int pairs = (int)(kRotateBytes / (sb + db)) + 1;
    Ring srcs((size_t)sb, pairs), dsts((size_t)db, pairs);
    auto f = [&](int i, hipStream_t s) {
        const int j = i % pairs;
        if (resize_linear(srcs.p[j], dsts.p[j], 1, 2160, 3840, 3, MI_RESIZE_U8, 1080, 1920, s) != 0)
            exit(3);
    };
    for (int S : {1, 2, 3, 4}) {
        const double us = time_us(f, 400, S, st);
        printf("{\"section\": \"resize_4k_rgb\", \"streams\": %d, \"us_per_frame\": %.3f, "
               "\"GBps\": %.1f, \"frac_of_peak\": %.4f, \"Gpix_s\": %.1f}\n",
               S, us, (sb + db) / (us * 1e3), (sb + db) / (us * 1e3) / kPeakGBps,
               2073600.0 / (us * 1e3));
    }
}

// The exact 2:1 RGB resize at width 3840 and several heights: time against
// output rows, fitted by least squares to a fixed cost plus a cost per row.
// The slope gives the rate at which the kernel moves bytes once it runs
// (28,800 bytes per output row); the intercept the cost no frame size
// amortises (launch, ramp and drain).
void resize_rows_fit(hipStream_t *st)
{
    std::vector<double> xs, ys;
    for (int dh : {540, 810, 1080, 1350, 1620}) {
        const long long sb = 2ll * dh * 3840 * 3, db = (long long)dh * 1920 * 3;
        const int pairs = (int)(kRotateBytes / (sb + db)) + 1;
        Ring srcs((size_t)sb, pairs), dsts((size_t)db, pairs);
        auto f = [&](int i, hipStream_t s) {
            const int j = i % pairs;
            if (resize_linear(srcs.p[j], dsts.p[j], 1, 2 * dh, 3840, 3, MI_RESIZE_U8, dh, 1920, s) != 0)
                exit(3);
        };
        const double us = time_us(f, 400, 1, st);
        xs.push_back(dh);
        ys.push_back(us);
        printf("{\"section\": \"resize_rgb_2to1_rows\", \"src\": [%d, 3840, 3], \"dst\": [%d, 1920], "
               "\"us\": %.3f, \"GBps\": %.1f}\n", 2 * dh, dh, us, (sb + db) / (us * 1e3));
    }
    const double n = xs.size();
    double sx = 0, sy = 0, sxx = 0, sxy = 0;
    for (size_t i = 0; i < xs.size(); ++i) {
        sx += xs[i];
        sy += ys[i];
        sxx += xs[i] * xs[i];
        sxy += xs[i] * ys[i];
    }
    const double slope = (n * sxy - sx * sy) / (n * sxx - sx * sx);   // us per output row
    const double icpt = (sy - slope * sx) / n;
    const double marginal = 28800.0 / (slope * 1e3);                 // GB/s
    printf("{\"section\": \"resize_rgb_2to1_rows_fit\", \"fixed_us\": %.3f, \"ns_per_output_row\": "
           "%.4f, \"marginal_GBps\": %.1f, \"marginal_frac_of_peak\": %.4f, "
           "\"4k_predicted_us\": %.3f, \"marginal_GBps_needed_for_70pct_at_4k_with_this_fixed_cost\": "
           "%.1f}\n",
           icpt, slope * 1e3, marginal, marginal / kPeakGBps, icpt + 1080 * slope,
           31104000.0 / ((31104000.0 / (0.7 * kPeakGBps * 1e3) - icpt) * 1e3));
}

// The exact 2x one-channel resize (1080 x 1920 -> 2160 x 3840) beside the
// stand-ins above and a copy of the same bytes split evenly between reads
// and writes.
void up2_byte_mix(hipStream_t *st)
{
    const long long sb = (long long)kU2H * kU2W, db = 4 * sb;
    const int pairs = (int)(kRotateBytes / (sb + db)) + 1;
    Ring srcs((size_t)sb, pairs), dsts((size_t)db, pairs);
    const unsigned wgs = kU2Segs * kU2GapGroups;
    auto report = [&](const char *what, double us, long long bytes) {
        printf("{\"section\": \"up2x_byte_mix\", \"what\": \"%s\", \"bytes\": %lld, \"us\": %.3f, "
               "\"GBps\": %.1f, \"frac_of_peak\": %.4f}\n",
               what, bytes, us, bytes / (us * 1e3), bytes / (us * 1e3) / kPeakGBps);
    };
    auto wo = [&](int i, hipStream_t s) {
        hipLaunchKernelGGL(up2_standin<false>, dim3(wgs), dim3(256), 0, s, srcs.p[i % pairs],
                           dsts.p[i % pairs]);
    };
    report("stand-in, writes only (8.29 MB)", time_us(wo, 400, 1, st), db);
    auto rw = [&](int i, hipStream_t s) {
        hipLaunchKernelGGL(up2_standin<true>, dim3(wgs), dim3(256), 0, s, srcs.p[i % pairs],
                           dsts.p[i % pairs]);
    };
    report("stand-in, both source rows read then written", time_us(rw, 400, 1, st), sb + db);
    auto lin = [&](int i, hipStream_t s) {
        if (resize_linear(srcs.p[i % pairs], dsts.p[i % pairs], 1, kU2H, kU2W, 1, MI_RESIZE_U8,
                          2 * kU2H, 2 * kU2W, s) != 0)
            exit(3);
    };
    report("resize_linear 2x", time_us(lin, 400, 1, st), sb + db);
    auto nn = [&](int i, hipStream_t s) {
        if (resize_nearest(srcs.p[i % pairs], dsts.p[i % pairs], 1, kU2H, kU2W, 1, MI_RESIZE_U8,
                           2 * kU2H, 2 * kU2W, s) != 0)
            exit(3);
    };
    report("resize_nearest 2x", time_us(nn, 400, 1, st), sb + db);
    // the same-bytes copy: (sb + db) / 2 each way, from the destinations
    // (each at least that large) into the sources' ring of the same count
    const long long half = (sb + db) / 2;
    Ring other((size_t)half, pairs);
    auto cp = [&](int i, hipStream_t s) {
        if (resize_copy_bytes(dsts.p[i % pairs], other.p[(i + 1) % pairs], half, s) != 0) exit(2);
    };
    report("copy of the same bytes, half read and half written", time_us(cp, 400, 1, st), sb + db);
}

// The float RGBA resize 4320 x 7680 -> 5927 x 3153 (rows enlarge 1.372x,
// columns shrink 2.436x) beside the stand-in with its byte mix (every
// source byte read once, every output byte written once) and a copy of the
// same bytes split evenly between reads and writes.  Two buffer pairs of
// 830 MB rotate, so no launch finds its source in the Infinity Cache.
void rgbaf_byte_mix(hipStream_t *st)
{
    constexpr int H = 4320, W = 7680, DH = 5927, DW = 3153;
    const long long sb = 16ll * H * W, db = 16ll * DH * DW;
    const int pairs = 2;
    Ring srcs((size_t)sb, pairs), dsts((size_t)db, pairs);
    auto report = [&](const char *what, double us, long long bytes) {
        printf("{\"section\": \"rgbaf_byte_mix\", \"what\": \"%s\", \"bytes\": %lld, \"us\": %.3f, "
               "\"GBps\": %.1f, \"frac_of_peak\": %.4f}\n",
               what, bytes, us, bytes / (us * 1e3), bytes / (us * 1e3) / kPeakGBps);
    };
    const long long ns16 = sb / 16, nd16 = db / 16;
    auto standin = [&](auto kernel, int loads, const char *what) {
        if (ns16 % (256 * loads) != 0) exit(4);
        const unsigned groups = (unsigned)(ns16 / (256 * loads));
        auto mix = [&](int i, hipStream_t s) {
            hipLaunchKernelGGL(kernel, dim3(groups), dim3(256), 0, s,
                               (const u32x4 *)srcs.p[i % pairs], (u32x4 *)dsts.p[i % pairs], nd16);
        };
        report(what, time_us(mix, 40, 1, st), sb + db);
    };
    standin(mix_standin<4>, 4, "stand-in, source read once and output written once, 4 loads per lane");
    standin(mix_standin<8>, 8, "stand-in, source read once and output written once, 8 loads per lane");
    standin(mix_standin<16>, 16, "stand-in, source read once and output written once, 16 loads per lane");
    auto rs = [&](int i, hipStream_t s) {
        if (resize_linear(srcs.p[i % pairs], dsts.p[i % pairs], 1, H, W, 4, MI_RESIZE_F32, DH, DW,
                          s) != 0)
            exit(3);
    };
    report("resize_linear float RGBA", time_us(rs, 40, 1, st), sb + db);
    // the same-bytes copy: (sb + db) / 2 each way, from the sources (each
    // larger than that) into a ring of its own
    const long long half = (sb + db) / 2;
    Ring other((size_t)half, pairs);
    auto cp = [&](int i, hipStream_t s) {
        if (resize_copy_bytes(srcs.p[i % pairs], other.p[(i + 1) % pairs], half, s) != 0) exit(2);
    };
    report("copy of the same bytes, half read and half written", time_us(cp, 40, 1, st), sb + db);
}

void trace_4k(hipStream_t *st)
{
    const long long sb = 24883200, db = 6220800;
    const int pairs = (int)(kRotateBytes / (sb + db)) + 1;
    Ring srcs((size_t)sb, pairs), dsts((size_t)db, pairs);
    const unsigned items = kTrSegs * (kTrH / 2), wgs = items / 2;
    unsigned long long *tr;
    CK(hipMalloc(&tr, 16ull * items));
    CK(hipMemset(tr, 0, 16ull * items));
    // the traced launch sits among back-to-back launches of its own kind
    hold(st[0], 40);
    for (int i = 0; i < 40; ++i)
        hipLaunchKernelGGL(traced_half_rgb, dim3(wgs), dim3(128), 0, st[0], srcs.p[i % pairs],
                           dsts.p[i % pairs], tr);
    CK(hipStreamSynchronize(st[0]));
    std::vector<unsigned long long> h(2 * items);
    CK(hipMemcpy(h.data(), tr, 16ull * items, hipMemcpyDeviceToHost));
    CK(hipFree(tr));
    const double ns = 1e6 / g_wall_khz;
    unsigned long long t0 = ~0ull, t1 = 0, last_start = 0;
    std::vector<double> dur;
    for (unsigned i = 0; i < items; ++i) {
        t0 = std::min(t0, h[2 * i]);
        t1 = std::max(t1, h[2 * i + 1]);
        last_start = std::max(last_start, h[2 * i]);
        dur.push_back((double)(h[2 * i + 1] - h[2 * i]) * ns);
    }
    std::sort(dur.begin(), dur.end());
    printf("{\"section\": \"trace_4k_rgb_standin\", \"waves\": %u, \"first_start_to_last_start_ns\": "
           "%.0f, \"first_start_to_last_end_ns\": %.0f, \"wave_ns_p10\": %.0f, \"wave_ns_p50\": "
           "%.0f, \"wave_ns_p90\": %.0f, \"wave_ns_max\": %.0f}\n",
           items, (last_start - t0) * ns, (t1 - t0) * ns, dur[items / 10], dur[items / 2],
           dur[9 * items / 10], dur.back());
    // wave starts and ends per 500 ns
    std::vector<int> hs(24), he(24);
    for (unsigned i = 0; i < items; ++i) {
        hs[std::min<size_t>(23, (size_t)((h[2 * i] - t0) * ns / 500))]++;
        he[std::min<size_t>(23, (size_t)((h[2 * i + 1] - t0) * ns / 500))]++;
    }
    printf("{\"section\": \"trace_4k_rgb_standin_histogram\", \"bin_ns\": 500, \"starts\": [");
    for (int b = 0; b < 24; ++b) printf("%s%d", b ? ", " : "", hs[b]);
    printf("], \"ends\": [");
    for (int b = 0; b < 24; ++b) printf("%s%d", b ? ", " : "", he[b]);
    printf("]}\n");
}

}  // namespace

int main(int argc, char **argv)
{
    // optional arguments name the sections to run (all by default)
    auto want = [&](const char *name) {
        if (argc < 2) return true;
        for (int i = 1; i < argc; ++i)
            if (std::string(argv[i]) == name) return true;
        return false;
    };
    CK(hipDeviceGetAttribute(&g_wall_khz, hipDeviceAttributeWallClockRate, 0));
    hipStream_t st[4];
    for (auto &s : st) CK(hipStreamCreateWithFlags(&s, hipStreamNonBlocking));
    const struct { const char *name; void (*run)(hipStream_t *); } sections[] = {
        {"copy_vs_size", copy_vs_size},   {"empty_grid", empty_grids},
        {"read_only", read_only_stream},  {"resize_4k_rgb", resize_4k},
        {"resize_rgb_2to1_rows", resize_rows_fit}, {"trace_4k_rgb_standin", trace_4k},
        {"up2x_byte_mix", up2_byte_mix}, {"rgbaf_byte_mix", rgbaf_byte_mix}};
    for (const auto &sec : sections) {
        if (!want(sec.name)) continue;
        sec.run(st);
        fflush(stdout);
    }
    for (auto &s : st) CK(hipStreamDestroy(s));
    return 0;
}
