// stubs.h -- what the stub launchers (stubs.cpp) record.
#pragma once

struct HostLaunchLog {
    long long split_valu = 0, split_mfma = 0, balanced = 0, combine = 0, pieces = 0;
    // when set, balanced launches check their descriptors end before this byte
    const char *workspace_end = nullptr;
};

HostLaunchLog &host_launch_log();
