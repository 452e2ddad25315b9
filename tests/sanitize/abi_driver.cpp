// Drives the host-side validation of the library's C ABI (include/ssm_scan.h)
// for a build whose host code carries AddressSanitizer and
// UndefinedBehaviorSanitizer (test infrastructure: tests/test_sanitize_cpu.py
// compiles and runs it). Every call below is refused before any launch, so the
// device addresses it passes are never dereferenced and no GPU is needed: the
// run exercises descriptor checks, size arithmetic (including sizes whose byte
// counts overflow), alignment and overlap tests, workspace sizing and the
// status strings. It also checks that each call returns the documented status.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ssm_scan.h"

namespace {

int failures = 0;

void expect(int got, int want, const char *what, int line) {
    if (got != want) {
        fprintf(stderr, "FAILED line %d: %s returned %d, expected %d\n", line, what, got, want);
        ++failures;
    }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

constexpr uintptr_t GB = uintptr_t(1) << 30;
void *at(uintptr_t a) { return reinterpret_cast<void *>(a); }
float *fat(uintptr_t a) { return reinterpret_cast<float *>(a); }

ssm_scan_desc desc(int64_t b = 2, int64_t L = 100, int64_t d = 64, int64_t N = 16, int dtype = SSM_BF16) {
    ssm_scan_desc s;
    memset(&s, 0, sizeof s);
    s.batch = b; s.seqlen = L; s.dim = d; s.dstate = N; s.dtype = dtype; s.disc = SSM_DISC_EULER;
    return s;
}

int scan(const ssm_scan_desc *d, uintptr_t u = 1 * GB, uintptr_t y = 8 * GB, uintptr_t hl = 9 * GB,
         uintptr_t ws = 11 * GB, size_t ws_bytes = size_t(1) << 30, uintptr_t h0 = 0) {
    return ssm_scan_fwd(d, at(u), at(2 * GB), fat(3 * GB), at(4 * GB), at(5 * GB), fat(6 * GB), at(7 * GB),
                        fat(h0), at(y), fat(hl), at(ws), ws_bytes, nullptr);
}

int bwd(const ssm_scan_desc *d, uintptr_t du = 9 * GB, uintptr_t dA = 11 * GB, uintptr_t dB = 12 * GB,
        uintptr_t ws = 16 * GB, size_t ws_bytes = size_t(1) << 30) {
    return ssm_scan_bwd(d, at(1 * GB), at(2 * GB), fat(3 * GB), at(4 * GB), at(5 * GB), fat(6 * GB), at(7 * GB),
                        nullptr, at(8 * GB), nullptr, at(du), at(10 * GB), fat(dA), fat(dB), fat(13 * GB),
                        fat(14 * GB), at(15 * GB), nullptr, nullptr, nullptr, nullptr, at(ws), ws_bytes, nullptr);
}

int decode(int64_t b, int64_t N, int dtype, uintptr_t x = 1 * GB, uintptr_t h = 8 * GB, uintptr_t y = 9 * GB) {
    return ssm_state_update(b, 64, N, dtype, SSM_DISC_EULER, at(x), at(2 * GB), nullptr, 0, fat(3 * GB), at(4 * GB),
                            at(5 * GB), fat(6 * GB), at(7 * GB), fat(h), at(y), nullptr);
}

ssm_ssd_desc sdesc(int64_t b = 2, int64_t L = 100, int H = 4, int P = 64, int G = 1, int N = 128) {
    ssm_ssd_desc s;
    memset(&s, 0, sizeof s);
    s.batch = b; s.seqlen = L; s.nheads = H; s.headdim = P; s.ngroups = G; s.dstate = N;
    s.dtype = SSM_BF16; s.disc = SSM_DISC_EULER;
    return s;
}

int ssd(const ssm_ssd_desc *d, uintptr_t x = 1 * GB, uintptr_t y = 8 * GB, uintptr_t hl = 9 * GB) {
    return ssm_ssd_fwd(d, at(x), at(2 * GB), fat(3 * GB), at(4 * GB), at(5 * GB), fat(6 * GB), at(7 * GB), nullptr,
                       at(y), fat(hl), nullptr);
}

}  // namespace

int main() {
    // forward scan
    ssm_scan_desc d = desc();
    EXPECT(scan(nullptr), SSM_ERR_NULL);
    ssm_scan_desc bad = desc(-1);
    EXPECT(scan(&bad), SSM_ERR_SHAPE);
    bad = desc(2, 100, 64, 16, 7);
    EXPECT(scan(&bad), SSM_ERR_DTYPE);
    bad = desc(2, 100, 64, 65);
    EXPECT(scan(&bad), SSM_ERR_UNSUPPORTED);
    bad = desc(int64_t(1) << 40, int64_t(1) << 30, 1 << 20);   // byte counts overflow
    EXPECT(scan(&bad), SSM_ERR_SHAPE);
    EXPECT((int)ssm_scan_workspace_size(&bad), 0);
    EXPECT(scan(&d, 1 * GB + 1), SSM_ERR_ALIGN);
    EXPECT(scan(&d, 1 * GB, 1 * GB + 64), SSM_ERR_ALIAS);        // y over u
    EXPECT(scan(&d, 1 * GB, 8 * GB, 9 * GB, 11 * GB, 16), SSM_ERR_WORKSPACE);
    EXPECT(scan(&d, 1 * GB, 8 * GB, 9 * GB, 11 * GB + 64), SSM_ERR_ALIGN);
    EXPECT(scan(&d, 1 * GB, 8 * GB, 9 * GB, 0, 0), SSM_ERR_WORKSPACE);
    EXPECT(scan(&d, 1 * GB, 8 * GB, 10 * GB + 4, 11 * GB, size_t(1) << 30, 10 * GB), SSM_ERR_ALIAS);
    ssm_scan_desc empty = desc(0);
    EXPECT(scan(&empty), SSM_OK);
    ssm_scan_tuning tun{3, 1};
    EXPECT(ssm_scan_fwd_tuned(&d, at(GB), at(2 * GB), fat(3 * GB), at(4 * GB), at(5 * GB), nullptr, nullptr, nullptr,
                              at(8 * GB), nullptr, at(11 * GB), size_t(1) << 30, &tun, nullptr),
           SSM_ERR_UNSUPPORTED);
    ssm_scan_tuning plan{};
    EXPECT(ssm_scan_plan(&d, &plan), SSM_OK);
    EXPECT(ssm_scan_plan(&d, nullptr), SSM_ERR_NULL);
    // the convolution prologue: its taps are required, its u needs workspace
    ssm_scan_desc conv = desc();
    conv.conv_width = 4;
    EXPECT(scan(&conv), SSM_ERR_NULL);
    conv.conv_weight = fat(17 * GB);
    EXPECT(scan(&conv, 1 * GB, 8 * GB, 9 * GB, 11 * GB, ssm_scan_workspace_size(&conv) - 1), SSM_ERR_WORKSPACE);
    conv.conv_width = 5;
    EXPECT(scan(&conv), SSM_ERR_UNSUPPORTED);
    // the forward without allocation: scratch limit checked before any HIP call
    ssm_scan_desc big = desc(64, int64_t(1) << 20, 4096, 64);
    EXPECT(ssm_scan_fwd_noalloc(&big, at(GB), at(2 * GB), fat(3 * GB), at(4 * GB), at(5 * GB), nullptr, nullptr,
                                nullptr, at(8 * GB), nullptr, nullptr),
           SSM_ERR_SCRATCH);
    EXPECT(ssm_scan_fwd_noalloc(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                nullptr, nullptr, nullptr),
           SSM_ERR_NULL);

    // backward and the training pair
    EXPECT(bwd(nullptr), SSM_ERR_NULL);
    bad = desc(2, 100, 64, 65);
    EXPECT(bwd(&bad), SSM_ERR_UNSUPPORTED);
    EXPECT(bwd(&d, 9 * GB + 1), SSM_ERR_ALIGN);
    EXPECT(bwd(&d, 1 * GB + 64), SSM_ERR_ALIAS);                 // du over u
    EXPECT(bwd(&d, 9 * GB, 11 * GB, 11 * GB + 4), SSM_ERR_ALIAS); // dB over dA
    EXPECT(bwd(&d, 9 * GB, 11 * GB, 12 * GB, 16 * GB, 16), SSM_ERR_WORKSPACE);
    const size_t bwd_need = ssm_scan_bwd_workspace_size(&d);
    EXPECT(bwd_need > ssm_scan_workspace_size(&d) ? 1 : 0, 1);
    EXPECT(ssm_scan_fwd_save(&d, at(GB), at(2 * GB), fat(3 * GB), at(4 * GB), at(5 * GB), fat(6 * GB), at(7 * GB),
                             nullptr, at(8 * GB), fat(9 * GB), at(11 * GB), bwd_need - 1, nullptr),
           SSM_ERR_WORKSPACE);
    EXPECT(ssm_scan_bwd_saved(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                              nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                              nullptr, nullptr, nullptr, nullptr, 0, nullptr),
           SSM_ERR_NULL);

    // decode step
    EXPECT(decode(-1, 16, SSM_BF16), SSM_ERR_SHAPE);
    EXPECT(decode(4, 80, SSM_BF16), SSM_ERR_UNSUPPORTED);
    EXPECT(decode(4, 16, 9), SSM_ERR_DTYPE);
    EXPECT(decode(4, 16, SSM_BF16, 1 * GB + 1), SSM_ERR_ALIGN);
    EXPECT(decode(4, 16, SSM_BF16, 1 * GB, 8 * GB, 8 * GB + 64), SSM_ERR_ALIAS);   // y inside h
    EXPECT(decode(4, 16, SSM_BF16, 1 * GB, 0), SSM_ERR_NULL);
    EXPECT(decode(0, 16, SSM_BF16), SSM_OK);

    // Mamba-2 SSD layer and its decode step
    ssm_ssd_desc s = sdesc();
    EXPECT(ssd(nullptr), SSM_ERR_NULL);
    ssm_ssd_desc sb = sdesc(2, 100, 6, 64, 4);
    EXPECT(ssd(&sb), SSM_ERR_SHAPE);
    sb = sdesc(2, 100, 4, 48);
    EXPECT(ssd(&sb), SSM_ERR_UNSUPPORTED);
    sb = sdesc(int64_t(1) << 40, int64_t(1) << 30);
    EXPECT(ssd(&sb), SSM_ERR_SHAPE);
    EXPECT(ssd(&s, 1 * GB + 8), SSM_ERR_ALIGN);
    EXPECT(ssd(&s, 1 * GB, 1 * GB + 64), SSM_ERR_ALIAS);
    ssm_ssd_desc s1 = sdesc(2, 2);
    EXPECT(ssm_ssd_state_update(&s1, at(GB), at(2 * GB), fat(3 * GB), at(4 * GB), at(5 * GB), nullptr, nullptr,
                                fat(8 * GB), at(9 * GB), nullptr),
           SSM_ERR_SHAPE);

    // every status has its own description
    for (int st = SSM_ERR_SCRATCH; st <= SSM_OK; ++st)
        if (strcmp(ssm_status_string(st), "unknown status") == 0) {
            fprintf(stderr, "FAILED: status %d has no description\n", st);
            ++failures;
        }
    if (strcmp(ssm_status_string(12345), "unknown status") != 0) ++failures;

    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("library host validation sanitizer run: all calls refused as documented\n");
    return 0;
}
