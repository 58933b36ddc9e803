// host_stubs.h -- what the stand-in launchers of host_stubs.cpp record.
#pragma once

#include "gdn_internal.h"

struct StubLog {
    int copies = 0, syncs = 0, verifies = 0, commits = 0, ancestors = 0;
    int branch_verifies = 0, accepts = 0, builds = 0, commit_verifies = 0;
    int verify_verdict = 0;   // written to every sequence's verify status
    int commit_verdict = 0;   // written to every sequence's commit status
    hipError_t launch_error = hipSuccess;
    gdn::VerifyArgs last_verify{};
    gdn::CommitArgs last_commit{};
    gdn::CommitPrev last_prev{};
};

extern StubLog g_stub;
