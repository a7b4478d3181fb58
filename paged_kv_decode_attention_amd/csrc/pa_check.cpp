// Host-side check of a cache write's slot mapping.  The write kernels trust
// the mapping (a duplicate slot races, a slot past the pool is skipped), so
// this is the debugging aid a caller runs on a host copy before the write.
#include <algorithm>
#include <cstdio>
#include <new>
#include <utility>
#include <vector>

#include "pa_internal.h"

extern "C" int pa_check_slot_mapping(const int64_t* slot_mapping, int num_tokens,
                                     int64_t num_slots) {
    char msg[200];
    if (num_tokens < 0 || num_slots < 0)
        return pa::report_error(PA_ERR_INVALID_ARG, "negative token or slot count");
    if (num_tokens > 0 && !slot_mapping)
        return pa::report_error(PA_ERR_INVALID_ARG, "null slot mapping");
    std::vector<std::pair<int64_t, int>> used;   // (slot, token), padding left out
    try {
        used.reserve(num_tokens);
    } catch (const std::bad_alloc&) {
        return pa::report_error(PA_ERR_INVALID_ARG, "out of host memory");
    }
    for (int i = 0; i < num_tokens; ++i) {
        const int64_t s = slot_mapping[i];
        if (s < 0) continue;
        if (s >= num_slots) {
            snprintf(msg, sizeof msg, "token %d: slot %lld is past the pool (%lld slots)", i,
                     (long long)s, (long long)num_slots);
            return pa::report_error(PA_ERR_INVALID_ARG, msg);
        }
        used.emplace_back(s, i);
    }
    std::sort(used.begin(), used.end());
    for (size_t k = 1; k < used.size(); ++k) {
        if (used[k].first == used[k - 1].first) {
            snprintf(msg, sizeof msg, "slot %lld given to tokens %d and %d",
                     (long long)used[k].first, used[k - 1].second, used[k].second);
            return pa::report_error(PA_ERR_INVALID_ARG, msg);
        }
    }
    return PA_OK;
}
