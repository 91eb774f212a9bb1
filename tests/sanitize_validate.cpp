// Drives every host-side argument check of the library with sweeps of extreme, null and
// aliased arguments, to be built with AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_abi.py builds and runs it).  Pointers are fake addresses that the checks only
// compare, never dereference.  Any undefined behaviour (signed overflow, bad shift, ...) or
// memory error aborts the run; every call must return a status code.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "validate.h"

using namespace s3d;

namespace {

uint64_t state = 0x9e3779b97f4a7c15ull;
uint64_t next() {                           // xorshift64*
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return state * 0x2545f4914f6cdd1dull;
}
template <class T, size_t N>
T pick(const T (&v)[N]) { return v[next() % N]; }

const int32_t kInts[] = {std::numeric_limits<int32_t>::min(), -65, -1, 0, 1, 2, 5, 7, 63, 64, 65, 128, 176,
                         1000, 1374, 1408, 2816, 5632, 8000, 8001, 12288, 12289, 16384, 65535, 65536,
                         1 << 20, 1 << 24, (1 << 30) + 1, std::numeric_limits<int32_t>::max()};
const float kFloats[] = {0.f, -0.f, 1.f, -1.f, 0.125f, 4.1588830833596715f, 1e-45f, 3.4e38f,
                         std::numeric_limits<float>::infinity(), -std::numeric_limits<float>::infinity(),
                         std::numeric_limits<float>::quiet_NaN()};
const uintptr_t kBases[] = {0, 16, 0x7f0000000000ull, 0x7f0000000100ull, 0x7f0000400000ull,
                            0x7f4000000000ull, 0x7f8000000000ull, UINTPTR_MAX - 4095};

const void* ptr() { return reinterpret_cast<const void*>(pick(kBases) + 16 * (next() % 4)); }
const float* fptr() { return static_cast<const float*>(ptr()); }
const int32_t* iptr() { return static_cast<const int32_t*>(ptr()); }
int dtype() { return static_cast<int>(next() % 4) - 1; }   // -1, 0 (F32), 1 (BF16), 2
sparse3d_layout layout() {
    sparse3d_layout l;
    l.frames = pick(kInts);
    l.tokens = pick(kInts);
    l.stride = pick(kInts);
    l.specials = pick(kInts);
    return l;
}
sparse3d_layout good(int32_t frames) { return sparse3d_layout{frames, 1374, 1408, 5}; }

long calls = 0, bad = 0;
void check(int st) {
    ++calls;
    if (st < SPARSE3D_OK || st > SPARSE3D_ERR_ALIAS) ++bad;
}

}  // namespace

int main() {
    for (int it = 0; it < 20000; ++it) {
        sparse3d_layout a = layout(), b = layout();
        const bool real = next() % 3 == 0;              // sometimes well-formed layouts
        if (real) {
            a = good(pick(kInts) & 1023);
            b = good(a.frames);
        }
        const sparse3d_layout* pa = next() % 16 ? &a : nullptr;
        const sparse3d_layout* pb = next() % 16 ? &b : nullptr;
        check(check_layout(pa));
        check(check_heads_dims(pick(kInts), pick(kInts), pick(kInts)));
        check(check_logit_params(pick(kFloats), pick(kFloats)));
        check(validate_tile_scores(ptr(), ptr(), next() % 2 ? ptr() : nullptr, dtype(), pick(kInts), 64, 64, pa,
                                   pb, fptr(), fptr(), next() % 2 ? fptr() : nullptr, fptr(),
                                   next() % 2 ? ptr() : nullptr, next() % 2 ? ptr() : nullptr));
        check(validate_select_topk(fptr(), pick(kInts), pick(kInts), pick(kInts), pick(kInts), pick(kInts),
                                   pick(kInts), iptr(), iptr(), pick(kInts)));
        check(validate_attn(next() % 2, ptr(), ptr(), ptr(), dtype(), pick(kInts), 64, 64, pa, pb, iptr(),
                            iptr(), pick(kInts), next() % 2 ? ptr() : nullptr, next() % 2 ? ptr() : nullptr,
                            ptr(), dtype(), next() % 2 ? fptr() : nullptr));
        sparse3d_sga sga{};
        sga.grid_h = pick(kInts);
        sga.grid_w = pick(kInts);
        sga.window = pick(kInts);
        sga.k_full = next() % 2 ? ptr() : nullptr;
        sga.v_full = next() % 2 ? ptr() : nullptr;
        sga.kmean = next() % 2 ? fptr() : nullptr;
        sga.vmean = next() % 2 ? fptr() : nullptr;
        sga.mean_bias = pick(kFloats);
        check(validate_sga(next() % 4 ? &sga : nullptr, dtype(), pick(kInts), 64, pa, pb, ptr(), dtype(),
                           fptr()));
        check(validate_discarded_mean(ptr(), ptr(), dtype(), pick(kInts), 64, pa, pick(kInts), pick(kInts),
                                      pick(kInts), fptr(), fptr()));
        check(validate_selection_transpose(iptr(), iptr(), pick(kInts), pick(kInts), pick(kInts), pick(kInts),
                                           iptr(), next() % 2 ? iptr() : nullptr));
        check(validate_attn_bwd(ptr(), ptr(), ptr(), ptr(), ptr(), fptr(), dtype(), pick(kInts), 64, 64, pa, pb,
                                iptr(), iptr(), pick(kInts), iptr(), iptr(), next() % 2 ? ptr() : nullptr,
                                next() % 2 ? ptr() : nullptr, pick(kFloats), pick(kFloats), fptr(), fptr(), fptr(),
                                fptr(), next() % 2 ? fptr() : nullptr, next() % 2 ? fptr() : nullptr));
        check(validate_cast(fptr(), static_cast<int64_t>(next()) >> (next() % 64), dtype(), ptr()));
        sparse3d_layout out{};
        check(subsample_layout(pa, pick(kInts), pick(kInts), pick(kInts), pick(kInts), next() % 8 ? &out : nullptr));
        check(validate_subsample(ptr(), ptr(), dtype(), pick(kInts), 64, pa, pick(kInts), pick(kInts), pick(kInts),
                                 ptr(), ptr(), pb));
        (void)dropped_per_frame(pick(kInts) & 0xffff, pick(kInts) & 0xffff, (pick(kInts) & 0xff) + 1);
    }
    // a well-formed call of each kind passes
    const sparse3d_layout g = good(8);
    const auto P = [](uintptr_t gib) { return reinterpret_cast<void*>(0x7f0000000000ull + (gib << 30)); };
    int ok = 0;
    ok += validate_tile_scores(P(0), P(1), nullptr, SPARSE3D_BF16, 16, 64, 64, &g, &g, (float*)P(2), (float*)P(3),
                               nullptr, (float*)P(4)) == SPARSE3D_OK;
    ok += validate_select_topk((float*)P(0), 16, 176, 176, 18, 22, 0, (int32_t*)P(1), (int32_t*)P(2), 40) ==
          SPARSE3D_OK;
    ok += validate_attn(true, P(0), P(1), P(2), SPARSE3D_BF16, 16, 64, 64, &g, &g, (int32_t*)P(3), (int32_t*)P(4),
                        40, nullptr, nullptr, P(5), SPARSE3D_F32, (float*)P(6)) == SPARSE3D_OK;
    ok += validate_attn_bwd(P(0), P(1), P(2), P(3), P(4), (float*)P(5), SPARSE3D_BF16, 16, 64, 64, &g, &g,
                            (int32_t*)P(6), (int32_t*)P(7), 40, (int32_t*)P(8), (int32_t*)P(9), P(10), P(11),
                            4.1588830833596715f, 0.125f, (float*)P(12), (float*)P(13), (float*)P(14),
                            (float*)P(15), (float*)P(16), (float*)P(17)) == SPARSE3D_OK;
    std::printf("calls %ld, outside the status codes %ld, well-formed accepted %d of 4\n", calls, bad, ok);
    return (bad == 0 && ok == 4) ? 0 : 1;
}
